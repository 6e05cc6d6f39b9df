// Gathered projection GEMMs with the layer's epilogues (gfx950).
//
// C = A_gathered * W^T: A rows are token rows picked by an index list (the
// candidates and fresh rows for K/V, the selected rows for Q), W rows are output
// features. The bf16 kernel uses v_mfma_f32_32x32x16_bf16 with fp32 accumulation;
// the fp32 kernel is a plain FMA tiling for fp32 workloads. Both stage the
// accumulator tile in LDS for an epilogue that works on whole heads, so that each
// rotation pair (i, i + d/2) sits in one thread; the bf16 kernel's items cover both
// 128-column blocks of its 256-column tile (shared rotation coefficients, one
// round trip of loads), the fp32 kernel and the encode mode go block by block.
#include <type_traits>

#include "kernels.hpp"

namespace srp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBN = 128;
constexpr int kLDC = kBN + 4;  // fp32 kernel staging stride

// ------------------------------------------------------------------------- //
// epilogue
// ------------------------------------------------------------------------- //
// Per-row metadata of a tile (token row, position, position delta), loaded
// once per tile so the epilogue's global loads do not wait on each other.
struct EpiRow {
  int row, pos, delta, cache;  // token row, position, rotation index, cache row
};

template <int MODE, int ROWS>
__device__ __forceinline__ void load_row_meta(EpiRow *meta, int m0, int M, const GemmArgs &g) {
  for (int r = threadIdx.x; r < ROWS; r += blockDim.x) {
    const int m = m0 + r;
    EpiRow e{-1, 0, kFresh, -1};
    if (m < M) {
      e.row = (MODE != EPI_ENC && g.a_rows) ? g.a_rows[m] : m;
      e.pos = g.positions[e.row];
      if (MODE == EPI_KV || MODE == EPI_V) e.delta = g.row_delta[e.row];
      if (MODE == EPI_KV || MODE == EPI_V || MODE == EPI_QK) e.cache = g.row_slot ? g.row_slot[e.row] : e.row;
    }
    meta[r] = e;
  }
}

__device__ __forceinline__ void rope_coef(const RopeTable &t, int p, int i0, float c[4], float s[4]) {
  int ap = p < 0 ? -p : p;
  ap = ap < t.max_pos ? ap : t.max_pos - 1;  // never read past the table
  ld4(t.cos_t + (size_t)ap * t.half + i0, c);
  ld4(t.sin_t + (size_t)ap * t.half + i0, s);
  if (p < 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) s[k] = -s[k];
  }
}

__device__ __forceinline__ void rotate4(float a[4], float b[4], const float c[4], const float s[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x = a[k], y = b[k];
    a[k] = x * c[k] - y * s[k];
    b[k] = y * c[k] + x * s[k];
  }
}

// Works through ROWS staged rows x 128 columns (Cs[r * ldc + c], fp32; block
// row r is tile row m_base + r, its metadata meta[r]) with NT threads: item =
// (row, head unit, 4 rotation pairs). Items go in batches of B whose global
// loads (rotation coefficients, cached K/V) are all issued before any of the
// batch's stores. A head unit is a Q, K or V head by the mode and its column.
template <typename T, int ROWS, int MODE, int NT, int B>
__device__ __forceinline__ void epilogue(const float *Cs, int ldc, const EpiRow *meta, int m_base,
                                         int n0, const GemmArgs &g) {
  constexpr int ITEMS = ROWS * 16 / NT;
  static_assert(ROWS * 16 % NT == 0 && ITEMS % B == 0, "items split evenly");
  constexpr bool SCORE = MODE == EPI_KV || MODE == EPI_V;  // fresh K/V + deviation
  const int d = g.d, half = d >> 1;
  const int tpu = d >> 3;  // threads per head unit (4 pairs each)
  const int kvd = g.nkv * d, qd = g.nh * d;
  // part of the unit at global column nu (0 = Q, 1 = K, 2 = V) and its head index
  auto unit = [&](int nu, int &part, int &hidx) __attribute__((always_inline)) {
    if (MODE == EPI_Q) {
      part = 0;
      hidx = nu / d;
    } else if (MODE == EPI_QK) {
      part = nu < qd ? 0 : 1;
      hidx = (nu - (part ? qd : 0)) / d;
    } else if (MODE == EPI_V) {
      part = 2;
      hidx = nu / d;
    } else {
      part = nu < kvd ? 1 : 2;
      hidx = (nu - (part == 2 ? kvd : 0)) / d;
    }
  };
#pragma unroll 1
  for (int kb = 0; kb < ITEMS; kb += B) {
    float c1[B][4], s1[B][4], c2[B][4], s2[B][4], ca[B][4], cb[B][4];
    // loads of the batch
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int it = threadIdx.x + (kb + j) * NT;
      const int r = it >> 4, qq = it & 15;
      const int u = qq / tpu, t = qq - u * tpu;
      const int nu = n0 + u * d, i0 = t * 4;
      const EpiRow e = meta[r];
      const bool valid = e.row >= 0 && nu < g.N;
      int part, hidx;
      unit(nu, part, hidx);
      if (valid && part <= 1) rope_coef(g.rope, e.pos, i0, c1[j], s1[j]);
      if (SCORE && valid && e.delta != kFresh) {
        const T *c = (const T *)(part == 2 ? g.v_cache : g.k_cache) + (size_t)e.cache * kvd + hidx * d;
        ld4(c + i0, ca[j]);
        ld4(c + half + i0, cb[j]);
        if (part == 1) rope_coef(g.rope, e.delta, i0, c2[j], s2[j]);
      }
    }
    // compute and store
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int it = threadIdx.x + (kb + j) * NT;
      const int r = it >> 4, qq = it & 15;
      const int u = qq / tpu, t = qq - u * tpu;
      const int nu = n0 + u * d, i0 = t * 4;
      const int m = m_base + r;
      const EpiRow e = meta[r];
      const bool valid = e.row >= 0 && nu < g.N;
      int part, hidx;
      unit(nu, part, hidx);
      float a[4], b[4];
      const float *src = Cs + r * ldc + u * d;
#pragma unroll
      for (int k = 0; k < 4; ++k) { a[k] = src[i0 + k]; b[k] = src[half + i0 + k]; }
      float part_sum = 0.f;
      int slot = -1;
      if (valid) {
        if (part <= 1) rotate4(a, b, c1[j], s1[j]);
        if (part == 0) {
#pragma unroll
          for (int k = 0; k < 4; ++k) { a[k] *= g.q_scale; b[k] *= g.q_scale; }
          T *q = (T *)g.q_out + (size_t)m * qd + hidx * d;
          st4(q + i0, a);
          st4(q + half + i0, b);
        } else if (MODE == EPI_QK) {
          // fresh key of a selected row, straight into its cache row
          T *o = (T *)g.k_cache + (size_t)e.cache * kvd + hidx * d;
          st4(o + i0, a);
          st4(o + half + i0, b);
        } else if (MODE == EPI_ENC) {
          T *o = (T *)(part == 2 ? g.v_cache : g.k_cache) + (size_t)m * kvd + hidx * d;
          st4(o + i0, a);
          st4(o + half + i0, b);
        } else {
          T *f = (T *)g.fresh + (size_t)m * 2 * kvd + (part - 1) * kvd + hidx * d;
          st4(f + i0, a);
          st4(f + half + i0, b);
          slot = (part - 1) * g.nkv + hidx;
          if (e.delta != kFresh) {
            if (part == 1) {
              // positional recovery of the cached key, kept in fp32 for the
              // deviation and written back to the cache
              rotate4(ca[j], cb[j], c2[j], s2[j]);
              T *c = (T *)g.k_cache + (size_t)e.cache * kvd + hidx * d;
              st4(c + i0, ca[j]);
              st4(c + half + i0, cb[j]);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float x = a[k] - ca[j][k], y = b[k] - cb[j][k];
              part_sum += x * x + y * y;
            }
          }
        }
      }
      if (SCORE) {
        // fixed-order reduction over the head's tpu lanes (aligned groups)
        for (int o = 1; o < tpu; o <<= 1) part_sum += __shfl_xor(part_sum, o, 64);
        if (valid && t == 0) g.dev_part[(size_t)m * 2 * g.nkv + slot] = part_sum;
      }
    }
  }
}

// Projection modes other than the encode on a 256-column tile: each item covers
// the same (row, 4 rotation pairs) of both 128-column blocks, so the two blocks
// share the rotation coefficients and one round trip of loads.
template <typename T, int ROWS, int MODE, int NT, int B>
__device__ __forceinline__ void epilogue_pair(const float *Cs, int ldc, const EpiRow *meta, int m_base,
                                              int n0, const GemmArgs &g) {
  constexpr int ITEMS = ROWS * 16 / NT;
  static_assert(ROWS * 16 % NT == 0 && ITEMS % B == 0, "items split evenly");
  constexpr bool SCORE = MODE == EPI_KV || MODE == EPI_V;  // fresh K/V + deviation
  const int d = g.d, half = d >> 1;
  const int tpu = d >> 3;
  const int kvd = g.nkv * d, qd = g.nh * d;
#pragma unroll 1
  for (int kb = 0; kb < ITEMS; kb += B) {
    int r[B], u[B], t[B], part[B][2], hidx[B][2];
    bool valid[B][2], any_k[B], cached[B];
    EpiRow e[B];
    float c1[B][4], s1[B][4], c2[B][4], s2[B][4];
    uint2 ra[B][2], rb[B][2];  // cached bf16 values, widened where used
    static_assert(sizeof(T) == 2, "bf16 cache rows");
    // loads of the batch
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int it = threadIdx.x + (kb + j) * NT;
      r[j] = it >> 4;
      const int qq = it & 15;
      u[j] = qq / tpu;
      t[j] = qq - u[j] * tpu;
      const int i0 = t[j] * 4;
      e[j] = meta[r[j]];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int nu = n0 + h * kBN + u[j] * d;
        valid[j][h] = e[j].row >= 0 && nu < g.N;
        // part of the unit (0 = Q, 1 = K, 2 = V) and its head index
        if (MODE == EPI_Q) {
          part[j][h] = 0;
          hidx[j][h] = nu / d;
        } else if (MODE == EPI_QK) {
          part[j][h] = nu < qd ? 0 : 1;
          hidx[j][h] = (nu - (nu < qd ? 0 : qd)) / d;
        } else {
          part[j][h] = MODE == EPI_V ? 2 : (nu < kvd ? 1 : 2);
          hidx[j][h] = (nu - (part[j][h] == 2 && MODE == EPI_KV ? kvd : 0)) / d;
        }
      }
      // units roped at the row's position (Q and K)
      any_k[j] = (valid[j][0] && part[j][0] <= 1) || (valid[j][1] && part[j][1] <= 1);
      cached[j] = SCORE && e[j].delta != kFresh;
      if (any_k[j]) rope_coef(g.rope, e[j].pos, i0, c1[j], s1[j]);
      if (MODE == EPI_KV && any_k[j] && cached[j]) rope_coef(g.rope, e[j].delta, i0, c2[j], s2[j]);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (valid[j][h] && cached[j]) {
          const T *c = (const T *)(part[j][h] == 2 ? g.v_cache : g.k_cache) + (size_t)e[j].cache * kvd +
                       hidx[j][h] * d;
          ra[j][h] = *reinterpret_cast<const uint2 *>(c + i0);
          rb[j][h] = *reinterpret_cast<const uint2 *>(c + half + i0);
        }
    }
    // compute and store
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i0 = t[j] * 4;
      const int m = m_base + r[j];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float a[4], b[4];
        const float *src = Cs + r[j] * ldc + h * kBN + u[j] * d;
#pragma unroll
        for (int k = 0; k < 4; ++k) { a[k] = src[i0 + k]; b[k] = src[half + i0 + k]; }
        float part_sum = 0.f;
        if (valid[j][h] && !SCORE) {
          rotate4(a, b, c1[j], s1[j]);
          if (part[j][h] == 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) { a[k] *= g.q_scale; b[k] *= g.q_scale; }
            T *q = (T *)g.q_out + (size_t)m * qd + hidx[j][h] * d;
            st4(q + i0, a);
            st4(q + half + i0, b);
          } else {
            // fresh key of a selected row, straight into its cache row
            T *o = (T *)g.k_cache + (size_t)e[j].cache * kvd + hidx[j][h] * d;
            st4(o + i0, a);
            st4(o + half + i0, b);
          }
        } else if (valid[j][h]) {
          if (part[j][h] == 1) rotate4(a, b, c1[j], s1[j]);
          T *f = (T *)g.fresh + (size_t)m * 2 * kvd + (part[j][h] - 1) * kvd + hidx[j][h] * d;
          st4(f + i0, a);
          st4(f + half + i0, b);
          if (cached[j]) {
            float ca[4], cb[4];
            ca[0] = __uint_as_float(ra[j][h].x << 16); ca[1] = __uint_as_float(ra[j][h].x & 0xffff0000u);
            ca[2] = __uint_as_float(ra[j][h].y << 16); ca[3] = __uint_as_float(ra[j][h].y & 0xffff0000u);
            cb[0] = __uint_as_float(rb[j][h].x << 16); cb[1] = __uint_as_float(rb[j][h].x & 0xffff0000u);
            cb[2] = __uint_as_float(rb[j][h].y << 16); cb[3] = __uint_as_float(rb[j][h].y & 0xffff0000u);
            if (part[j][h] == 1) {
              // positional recovery of the cached key, kept in fp32 for the
              // deviation and written back to the cache
              rotate4(ca, cb, c2[j], s2[j]);
              T *c = (T *)g.k_cache + (size_t)e[j].cache * kvd + hidx[j][h] * d;
              st4(c + i0, ca);
              st4(c + half + i0, cb);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float x = a[k] - ca[k], y = b[k] - cb[k];
              part_sum += x * x + y * y;
            }
          }
        }
        if (SCORE) {
          // fixed-order reduction over the head's tpu lanes (aligned groups)
          for (int o = 1; o < tpu; o <<= 1) part_sum += __shfl_xor(part_sum, o, 64);
          if (valid[j][h] && t[j] == 0)
            g.dev_part[(size_t)m * 2 * g.nkv + (part[j][h] - 1) * g.nkv + hidx[j][h]] = part_sum;
        }
      }
    }
  }
}

// Calls f(integral_constant<int, i>) for i = 0..N-1 (compile-time indices).
template <int N, typename F>
__device__ __forceinline__ void static_for_gemm(F &&f) {
  if constexpr (N > 0) {
    static_for_gemm<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// ------------------------------------------------------------------------- //
// tile scheduling: persistent loop, each XCD (blockIdx % 8) walks a contiguous
// range of tiles so the operand slabs its work-groups read stay in its L2
// ------------------------------------------------------------------------- //
struct TileIter {
  int x, loc, per_x, chunk, total;
  __device__ TileIter(int total_) : total(total_) {
    x = blockIdx.x & 7;
    loc = blockIdx.x >> 3;
    per_x = gridDim.x >> 3;
    chunk = (total + 7) >> 3;
  }
  __device__ int tile(int lt) const {
    int t = x * chunk + lt;
    return (lt < chunk && t < total) ? t : -1;
  }
};

// ------------------------------------------------------------------------- //
// bf16 MFMA kernel: BM x BN tile, WM x WN waves, each wave owning a
// (BM/WM) x (BN/WN) block of 32x32x16 MFMA tiles. Operand tiles of depth BK
// stream into an S-slot LDS ring in 1 KB pieces (1024 / (2 BK) whole row
// segments each): 256x256 tiles stage them through registers while the two
// wave groups take turns (the mainloop below), other tiles copy them with
// direct-to-LDS loads. Row segments of at least 128 bytes (BK >= 64) keep the copies at full rate;
// 64-byte segments (half cache lines) run at a third of it. With CH = BK / 8
// chunks of 16 bytes per row, chunk c of row r is stored at
// c ^ ((r / (16 / CH)) % CH): a 16-byte LDS read serves 16 lanes (64 banks) per
// cycle, the fragment reads put 16 consecutive rows in those lanes, and this
// layout gives them 16 different bank groups.
// ------------------------------------------------------------------------- //

template <int BM_, int BN_, int WM_, int WN_, int S_, int BK_>
struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, S = S_, BK = BK_;
  static constexpr int CH = BK / 8;    // 16-byte chunks per operand row
  static constexpr int RPC = 64 / CH;  // rows per 1 KB copy
  static constexpr int SWZ = 16 / CH;  // consecutive rows sharing a swizzle value
  static constexpr int WAVES = WM * WN, THREADS = 64 * WAVES;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int MI = TM / 32, NI = TN / 32;
  static constexpr int ATILE = BM * BK * 2, STAGE = (BM + BN) * BK * 2;
  static constexpr int ACOPY = BM / RPC, COPIES = (BM + BN) / RPC;
  static constexpr int CPW = COPIES / WAVES;  // copies per wave per tile
  static constexpr int EROWS = TM;            // rows staged per epilogue pass (one wave row)
  static constexpr int LDC = BN + 4;
  static constexpr int RING = S * STAGE, CS = EROWS * LDC * 4;
  static constexpr int SMEM = RING > CS ? RING : CS;
  static constexpr int PER_CU = THREADS >= 512 ? 1 : 2;  // resident work-groups per CU
  // epilogue load batch (items per thread): the other wave row's accumulators
  // are still live while the first row is finished, which leaves room for one
  static constexpr int EPI_B = 1;
  static_assert(COPIES % WAVES == 0 && ACOPY % WAVES == 0, "copies split evenly, A before B");
  static_assert(BN % kBN == 0, "the epilogue works on 128-column blocks");
};

// Tile order of the bf16 kernels: groups of gm row tiles, column-major inside a
// group. An XCD runs c = min(work-groups per XCD, its share of tiles) consecutive
// tiles at once; choosing gm to minimise gm + ceil(c / gm) makes them a near-square
// block, so each k-step the XCD's L2 fetches gm A slabs and ceil(c / gm) B slabs
// (row-major order fetches every B slab whenever a row of tiles is wider than c).
struct TileMap {
  int mt_n, nt_n, gm;
  __device__ TileMap(int mt_n_, int nt_n_, int whole, int grid) : mt_n(mt_n_), nt_n(nt_n_), gm(1) {
    const int per_x = grid >> 3, share = (whole + 7) >> 3;
    const int c = per_x < share ? per_x : share;
    int best = 1 << 30;
    for (int r = 1; r <= mt_n && r <= c; ++r) {
      const int cols = (c + r - 1) / r;
      if (cols > nt_n) continue;
      if (r + cols < best) best = r + cols, gm = r;
    }
  }
  __device__ void mn(int t, int &mt, int &nt) const {
    const int gsz = gm * nt_n, grp = t / gsz, idx = t - grp * gsz, r0 = grp * gm;
    const int gh = mt_n - r0 < gm ? mt_n - r0 : gm;
    nt = idx / gh;
    mt = r0 + (idx - nt * gh);
  }
};

// Work split: the full rounds of tiles (floor(T / P) per work-group) run whole;
// the R tiles of the last, partial round are split along K into s pieces each
// (s <= P / R), whose fp32 partial tiles a second kernel adds up and finishes
// with the epilogue. Both kernels derive the plan from the same numbers.
constexpr int kMaxSplit = 8;
struct SplitPlan {
  int tiles, full, tail, split;  // T, tiles run whole, tail tiles, pieces per tail tile
};
__host__ __device__ inline SplitPlan split_plan(int tiles, int grid, int part_cap) {
  SplitPlan sp{tiles, tiles, 0, 1};
  const int tail = tiles % grid;
  if (tail == 0 || part_cap <= 0) return sp;
  int s = grid / tail;
  s = s < kMaxSplit ? s : kMaxSplit;
  s = s < part_cap / tail ? s : part_cap / tail;
  if (s < 2) return sp;
  sp.full = tiles - tail;
  sp.tail = tail;
  sp.split = s;
  return sp;
}

template <int MODE, typename C>
__global__ __launch_bounds__(C::THREADS, C::PER_CU) void gemm_bf16_kernel(GemmArgs g) {
  static_assert(C::BM * C::BN <= kGemmPartFloats, "partial tiles fit their slots");
  static_assert(C::BK / 16 >= 3, "a stage's copies spread over three 16-deep steps");
  __shared__ __align__(16) char smem[C::SMEM];
  __shared__ EpiRow meta[C::BM];
  float *Cs = reinterpret_cast<float *>(smem);  // epilogue staging, EROWS x LDC fp32

  const int M = g.M_dev ? *g.M_dev : g.M_host;
  const int K = g.K, N = g.N;
  const int mt_n = (M + C::BM - 1) / C::BM, nt_n = (N + C::BN - 1) / C::BN;
  const SplitPlan sp = split_plan(mt_n * nt_n, gridDim.x, g.part_cap);
  const TileMap tm(mt_n, nt_n, sp.full, gridDim.x);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / C::WN, wn = w - wm * C::WN;
  const char *A = (const char *)g.A, *B = (const char *)g.B;
  const int KT = K / C::BK;
  const size_t rowb = (size_t)K * 2;
  // copy layout: lane covers row RPC*q + lrow and physical chunk lane % CH,
  // which holds logical chunk lchunk. This wave's copies are q = w + WAVES*j,
  // and the swizzle term of their rows depends on q only through w.
  const int lrow = lane / C::CH;
  const int lchunk = (lane % C::CH) ^ (((C::RPC * w + lrow) / C::SWZ) % C::CH);
  // fragment reads: lane holds row (lane % 32) of a 32-row block and k-values
  // 8 * (lane / 32) .. +8 of each 16-deep step
  const int fr = lane & 31, fk = lane >> 5;
  const uint32_t fswz = (fr / C::SWZ) % C::CH;
  floatx16 acc[C::MI][C::NI];
  // 256x256 tiles run the two wave groups in turns (below); the encode's epilogue
  // needs more registers than that schedule leaves, so it keeps the shared ring loop
  constexpr bool kPingPong = C::S == 2 && C::WAVES == 8 && C::WM == 2 && C::BK == 64 && MODE != EPI_ENC;

  // acc = A[m0.., k0*32 ..] * B[n0.., ..]^T over nk k-tiles; `pre` runs once the
  // first copies are in flight
  auto mainloop = [&](int m0, int n0, int k0, int nk, auto pre) __attribute__((always_inline)) {
    // copies are 1 KB operand pieces q of a stage, A's first; in the shared ring
    // loop wave w moves q = w + WAVES*j. Rows past M or N read a valid row (their
    // results are never stored).
    const int row0 = g.a_rows ? g.a_rows[m0] : m0;
    // source of copy q of the first k-tile (A copies first, then B)
    auto copy_src = [&](int q) __attribute__((always_inline)) -> const char * {
      if (q < C::ACOPY) {
        const int m = m0 + C::RPC * q + lrow;
        const int row = m < M ? (g.a_rows ? g.a_rows[m] : m) : row0;
        return A + (size_t)row * rowb + (size_t)k0 * (C::BK * 2) + lchunk * 16;
      }
      const int n = n0 + C::RPC * (q - C::ACOPY) + lrow;
      return B + (size_t)(n < N ? n : N - 1) * rowb + (size_t)k0 * (C::BK * 2) + lchunk * 16;
    };
    const char *src[C::CPW];
    if constexpr (!kPingPong) {
#pragma unroll
      for (int j = 0; j < C::CPW; ++j) src[j] = copy_src(w + C::WAVES * j);
    }
    auto issue = [&](int kt) __attribute__((always_inline)) {
      char *st = smem + (kt % C::S) * C::STAGE;
#pragma unroll
      for (int j = 0; j < C::CPW; ++j) dma16(src[j] + (size_t)kt * (C::BK * 2), st + (w + C::WAVES * j) * 1024);
    };
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int j = 0; j < C::NI; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    if constexpr (kPingPong) {
      // Waves 0-3 and 4-7 (one of each on every SIMD) take turns: while one group
      // runs the MFMAs of 32 of a stage's 64 k-values from fragments it already
      // holds, the other reads its fragments of the next 32 and moves operand data,
      // so neither LDS reads nor global loads sit in a wave's MFMA stream. Both
      // groups run the same stream (read, barrier, MFMAs, barrier), waves 4-7 one
      // barrier later; numbering phases 4kt + p, group 0 reads stage kt in phases
      // 4kt and 4kt+2, group 1 in 4kt+1 and 4kt+3.
      // Group 0 reads only the top 128 A rows of a stage and group 1 only the
      // bottom ones; both read all of B. So the three regions of a slot free at
      // different phases, and every read phase fills a quarter of a later stage
      // into a region already free: group 0 the first half of B (phase 4kt) and the
      // bottom of A (4kt+2) of stage kt+1, group 1 the second half of B of stage
      // kt+1 (4kt+1) and the top of A of stage kt+2 (4kt+3). Each wave stages both
      // of its sets in registers: a read phase stores one set, loaded two read
      // phases earlier, and loads it again for the next stage. Global loads plus
      // LDS stores move operand data faster than direct-to-LDS copies, and the
      // compiler counts these loads itself.
      static_assert(C::CPW == 8 && C::ACOPY == 32 && C::COPIES == 64, "four copies per set");
      const bool g0 = w < C::WAVES / 2;
      const int u = w & (C::WAVES / 2 - 1);
      // set 0: group 0 the first half of B, group 1 the second half; set 1: group 0
      // the bottom of A, group 1 the top. Set h holds copies qs[h] + u + 4i.
      const int qs0 = g0 ? C::ACOPY : C::ACOPY + C::ACOPY / 2;
      const int qs1 = g0 ? C::ACOPY / 2 : 0;
      // set 0 reads B rows n0.. of this tile: 32-bit byte offsets from the first;
      // set 1 reads gathered A rows: full pointers
      const char *Bt = B + (size_t)n0 * rowb;
      uint32_t so0[4];
      const char *pa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        so0[i] = (uint32_t)(copy_src(qs0 + u + 4 * i) - Bt);
        pa[i] = copy_src(qs1 + u + 4 * i);
      }
      auto spp = [&](int h, int i) __attribute__((always_inline)) -> const char * {
        return h ? pa[i] : Bt + so0[i];
      };
      auto advance = [&](int h, int i) __attribute__((always_inline)) {
        if (h) pa[i] += C::BK * 2;
        else so0[i] += C::BK * 2;
      };
      // direct copies of set h into the slot of stage kt (prologue only)
      auto copy_set = [&](int h, int kt) __attribute__((always_inline)) {
        char *st = smem + (kt % C::S) * C::STAGE + ((h ? qs1 : qs0) + u) * 1024;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dma16(spp(h, i), st + i * 4096);
          advance(h, i);
        }
      };
      // each set staged in four scalars (an array under these conditions would be
      // kept in scratch memory)
      uint4 a0 = {0, 0, 0, 0}, a1 = a0, a2 = a0, a3 = a0, b0 = a0, b1 = a0, b2 = a0, b3 = a0;
      auto load_set = [&](int h) __attribute__((always_inline)) {
        if (h == 0) {
          a0 = *reinterpret_cast<const uint4 *>(spp(0, 0));
          a1 = *reinterpret_cast<const uint4 *>(spp(0, 1));
          a2 = *reinterpret_cast<const uint4 *>(spp(0, 2));
          a3 = *reinterpret_cast<const uint4 *>(spp(0, 3));
        } else {
          b0 = *reinterpret_cast<const uint4 *>(spp(1, 0));
          b1 = *reinterpret_cast<const uint4 *>(spp(1, 1));
          b2 = *reinterpret_cast<const uint4 *>(spp(1, 2));
          b3 = *reinterpret_cast<const uint4 *>(spp(1, 3));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) advance(h, i);
      };
      auto write_set = [&](int h, int kt) __attribute__((always_inline)) {
        char *st = smem + (kt % C::S) * C::STAGE + ((h ? qs1 : qs0) + u) * 1024 + lane * 16;
        *reinterpret_cast<uint4 *>(st) = h ? b0 : a0;
        *reinterpret_cast<uint4 *>(st + 4096) = h ? b1 : a1;
        *reinterpret_cast<uint4 *>(st + 8192) = h ? b2 : a2;
        *reinterpret_cast<uint4 *>(st + 12288) = h ? b3 : a3;
      };
      bf16x8 af[2][C::MI], bfr[2][C::NI];
      auto read_half = [&](int kt, int h) __attribute__((always_inline)) {
        const char *as = smem + (kt % C::S) * C::STAGE, *bs = as + C::ATILE;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int ks = 2 * h + s;
          const uint32_t off = fr * (C::BK * 2) + (((2 * ks + fk) ^ fswz) * 16);
#pragma unroll
          for (int i = 0; i < C::MI; ++i)
            af[s][i] = *reinterpret_cast<const bf16x8 *>(as + (wm * C::TM + i * 32) * (C::BK * 2) + off);
#pragma unroll
          for (int j = 0; j < C::NI; ++j)
            bfr[s][j] = *reinterpret_cast<const bf16x8 *>(bs + (wn * C::TN + j * 32) * (C::BK * 2) + off);
        }
      };
      auto sync = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      };
      // set 1 is stored at the second read phase of stage kt for stage kt + ydelta
      const int ydelta = g0 ? 1 : 2;
      if (nk > 0) {
        copy_set(0, 0);
        copy_set(1, 0);
      }
      pre();
      if (!g0 && nk > 1) copy_set(1, 1);
      wait_vmcnt<0>();
      // the first staged stage of each set
      if (nk > 1) load_set(0);
      if (ydelta < nk) load_set(1);
      sync();
      if (!g0) sync();
      for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          read_half(kt, h);
          // set h: store its stage for this read phase, then load the one after
          const int tgt = h == 0 ? kt + 1 : kt + ydelta;
          if (tgt < nk) write_set(h, tgt);
          if (tgt + 1 < nk) load_set(h);
          // fragments read and staged stores done before the phase's barrier
          wait_lgkmcnt0();
          sync();
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < C::MI; ++i)
#pragma unroll
              for (int j = 0; j < C::NI; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s][i], bfr[s][j], acc[i][j], 0, 0, 0);
          sync();
        }
      }
      if (g0) sync();
    } else {
#pragma unroll
      for (int p = 0; p < C::S - 1; ++p)
        if (p < nk) issue(p);
      pre();
      for (int kt = 0; kt < nk; ++kt) {
        // this tile's copies are done once at most those of the later tiles
        // already in flight are outstanding
        const int later = min(nk - 1 - kt, C::S - 2);
        if (later >= 3) wait_vmcnt<3 * C::CPW>();
        else if (later == 2) wait_vmcnt<2 * C::CPW>();
        else if (later == 1) wait_vmcnt<C::CPW>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        // the slot of tile kt+S-1 was last read in iteration kt-1. Its copies go out
        // in three groups, before the first three 16-deep steps: issued all at once
        // they stall the waves' MFMA issue while the copy unit drains them, and the
        // last step's would land too late
        const bool copy_next = kt + C::S - 1 < nk;
        char *st_next = smem + ((kt + C::S - 1) % C::S) * C::STAGE;
        const char *as = smem + (kt % C::S) * C::STAGE, *bs = as + C::ATILE;
#pragma unroll
        for (int ks = 0; ks < C::BK / 16; ++ks) {
          if (ks < 3 && copy_next) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = (ks * C::CPW) / 3; j < ((ks + 1) * C::CPW) / 3; ++j)
              dma16(src[j] + (size_t)(kt + C::S - 1) * (C::BK * 2), st_next + (w + C::WAVES * j) * 1024);
            __builtin_amdgcn_sched_barrier(0);
          }
          const uint32_t off = fr * (C::BK * 2) + (((2 * ks + fk) ^ fswz) * 16);
          bf16x8 af[C::MI], bfr[C::NI];
#pragma unroll
          for (int i = 0; i < C::MI; ++i)
            af[i] = *reinterpret_cast<const bf16x8 *>(as + (wm * C::TM + i * 32) * (C::BK * 2) + off);
#pragma unroll
          for (int j = 0; j < C::NI; ++j)
            bfr[j] = *reinterpret_cast<const bf16x8 *>(bs + (wn * C::TN + j * 32) * (C::BK * 2) + off);
#pragma unroll
          for (int i = 0; i < C::MI; ++i)
#pragma unroll
            for (int j = 0; j < C::NI; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  };

  // 1. one K-piece of a tail tile: fp32 partial tile to its slot
  if (sp.split > 1 && (int)blockIdx.x < sp.tail * sp.split) {
    const int piece = blockIdx.x;
    const int tile = sp.full + piece / sp.split, j = piece - (piece / sp.split) * sp.split;
    int mt, nt;
    tm.mn(tile, mt, nt);
    const int k0 = (int)((long)KT * j / sp.split), k1 = (int)((long)KT * (j + 1) / sp.split);
    mainloop(mt * C::BM, nt * C::BN, k0, k1 - k0, [] {});
    float *dst = g.part + (size_t)piece * kGemmPartFloats;
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
      for (int jj = 0; jj < C::NI; ++jj)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = wm * C::TM + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
          const int col = wn * C::TN + jj * 32 + (lane & 31);
          dst[row * C::BN + col] = acc[i][jj][e];
        }
    __syncthreads();  // the ring is free before the next tile's copies
  }

  // 2. whole tiles: each XCD walks a contiguous range of tiles in TileMap order
  const TileIter ti(sp.full);
  for (int lt = ti.loc;; lt += ti.per_x) {
    const int tile = ti.tile(lt);
    if (tile < 0) break;
    int mt, nt;
    tm.mn(tile, mt, nt);
    const int m0 = mt * C::BM, n0 = nt * C::BN;
    // the epilogue's row metadata loads while the first copies are in flight
    mainloop(m0, n0, 0, KT, [&] { load_row_meta<MODE, C::BM>(meta, m0, M, g); });
    if constexpr (MODE != EPI_ENC && C::BN == 2 * kBN && C::WM == 2 && C::MI == 4) {
      // each of two passes stages half of every wave's rows
      // (blocks i = 2p, 2p+1; D[row][col], row = 8*(e/4) + 4*(lane/32) + e%4), so
      // after the first pass half the accumulators are dead and the epilogue
      // items can go two per batch. Staged row r is tile row
      // (r / 64) * 128 + 64 p + r % 64.
      static_for_gemm<2>([&](auto P) __attribute__((always_inline)) {
        constexpr int p = decltype(P)::value;
        __syncthreads();  // the ring (or the previous pass) is no longer read
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int j = 0; j < C::NI; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int row = wm * 64 + ii * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
              const int col = wn * C::TN + j * 32 + (lane & 31);
              Cs[row * C::LDC + col] = acc[2 * p + ii][j][e];
            }
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
        for (int hr = 0; hr < 2; ++hr)
          epilogue_pair<uint16_t, 64, MODE, C::THREADS, 2>(Cs + hr * 64 * C::LDC, C::LDC, meta + hr * 128 + 64 * p,
                                                           m0 + hr * 128 + 64 * p, n0, g);
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
      // the epilogue runs once per wave row: the waves of row p stage their
      // accumulators (D[row][col], row = 8*(e/4) + 4*(lane/32) + e%4), then every
      // wave works through the staged rows one 128-column block at a time
#pragma unroll 1
      for (int p = 0; p < C::WM; ++p) {
        __syncthreads();  // the ring (or the previous pass) is no longer read
        if (wm == p) {
#pragma unroll
          for (int i = 0; i < C::MI; ++i)
#pragma unroll
            for (int j = 0; j < C::NI; ++j)
#pragma unroll
              for (int e = 0; e < 16; ++e) {
                const int row = i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
                const int col = wn * C::TN + j * 32 + (lane & 31);
                Cs[row * C::LDC + col] = acc[i][j][e];
              }
        }
        __syncthreads();
#pragma unroll 1
        for (int cb = 0; cb < C::BN / kBN; ++cb)
          epilogue<uint16_t, C::EROWS, MODE, C::THREADS, C::EPI_B>(Cs + cb * kBN, C::LDC, meta + p * C::TM,
                                                                  m0 + p * C::TM, n0 + cb * kBN, g);
      }
    }
    __syncthreads();
  }

  // 3. the Q projection leaves work-groups without tiles (fewer tiles than CUs)
  //    or finishing early: they build the attention's transposed V copy, chunks
  //    (64 keys, KV head) claimed from a counter, so it runs on otherwise idle CUs
  if constexpr (MODE == EPI_Q || MODE == EPI_QK) {
    if (g.vt_dst) {
      __shared__ int claim;
      constexpr int NCH = 4;  // chunks per claim, their loads in flight together
      const int rows_n = g.vt_stride / 64, n_chunks = rows_n * g.nkv;
      static_assert(NCH * 128 * kVtPitch * 2 <= C::SMEM, "the transpose tiles fit the ring");
      for (;;) {
        if (tid == 0) claim = atomicAdd(g.vt_ctr, NCH);
        __syncthreads();
        const int c = claim;
        if (c >= n_chunks) break;
        int r0[NCH], hg[NCH];
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
          const int ck = c + k < n_chunks ? c + k : c;
          hg[k] = ck / rows_n;
          r0[k] = (ck - hg[k] * rows_n) * 64;
        }
        const int n = n_chunks - c < NCH ? n_chunks - c : NCH;
        vt_chunks<C::THREADS, NCH>(n, r0, hg, g.vt_T, g.d, g.nkv, (const uint16_t *)g.vt_src, g.vt_slot,
                                   (uint16_t *)g.vt_dst, g.vt_stride, reinterpret_cast<uint16_t *>(smem));
        __syncthreads();  // the tiles and `claim` are reused by the next claim
      }
    }
  }
}

// Finishes the split tail tiles, one item (tail tile, block of 16 rows) at a
// time: adds the tile's K-piece partials and runs the epilogue on them. Small
// items keep many work-groups busy on a few tail tiles.
constexpr int kFixRows = 16;

// Cs[r][c] = sum over the split pieces of part[piece][r][c] for kFixRows rows of BN
// columns, 4 columns per thread and step (256 threads).
template <int NS, int BN, int LDC>
__device__ __forceinline__ void fix_sum(const float *base, int split, float *Cs) {
  constexpr int PER = kFixRows * BN / 4 / 256;
  static_assert(PER % 2 == 0, "column groups in pairs");
  for (int u0 = 0; u0 < PER; u0 += 2) {
    float4 v[NS][2];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int jj = j < split ? j : split - 1;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int idx = threadIdx.x + (u0 + u) * 256;
        const int r = idx / (BN / 4), c4 = (idx - r * (BN / 4)) * 4;
        v[j][u] = *reinterpret_cast<const float4 *>(base + (size_t)jj * kGemmPartFloats + (size_t)r * BN + c4);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const float wj = j < split ? 1.f : 0.f;
        acc.x += wj * v[j][u].x; acc.y += wj * v[j][u].y; acc.z += wj * v[j][u].z; acc.w += wj * v[j][u].w;
      }
      const int idx = threadIdx.x + (u0 + u) * 256;
      const int r = idx / (BN / 4), c4 = (idx - r * (BN / 4)) * 4;
      *reinterpret_cast<float4 *>(Cs + r * LDC + c4) = acc;
    }
  }
}

template <int MODE, typename C>
__global__ __launch_bounds__(256) void gemm_fixup_kernel(GemmArgs g) {
  constexpr int LDC = C::BN + 4;
  __shared__ __align__(16) float Cs[kFixRows * LDC];
  __shared__ EpiRow meta[kFixRows];
  const int M = g.M_dev ? *g.M_dev : g.M_host;
  const int mt_n = (M + C::BM - 1) / C::BM, nt_n = (g.N + C::BN - 1) / C::BN;
  const SplitPlan sp = split_plan(mt_n * nt_n, g.grid_main, g.part_cap);
  if (sp.split < 2) return;
  constexpr int RB = C::BM / kFixRows;
  const TileMap tm(mt_n, nt_n, sp.full, g.grid_main);
  // items (tail tile, block of kFixRows rows), strided over the grid
#pragma unroll 1
  for (int item = blockIdx.x; item < sp.tail * RB; item += gridDim.x) {
    const int ti = item / RB, rb = item - ti * RB;
    const int tile = sp.full + ti;
    int mt, nt;
    tm.mn(tile, mt, nt);
    const int m0 = mt * C::BM + rb * kFixRows, n0 = nt * C::BN;
    if (m0 >= M) continue;
    __syncthreads();  // the previous item's epilogue no longer reads meta or Cs
    load_row_meta<MODE, kFixRows>(meta, m0, M, g);
    // sum of the pieces into Cs: the loads of NS slots (NS = the split rounded up to
    // 2, 4 or 8; slots past the split clamped to a valid one and weighted 0) and of two
    // column groups are issued together, so the sum waits for one round trip
    const float *base = g.part + (size_t)ti * sp.split * kGemmPartFloats + (size_t)rb * kFixRows * C::BN;
    if (sp.split <= 2)
      fix_sum<2, C::BN, LDC>(base, sp.split, Cs);
    else if (sp.split <= 4)
      fix_sum<4, C::BN, LDC>(base, sp.split, Cs);
    else
      fix_sum<kMaxSplit, C::BN, LDC>(base, sp.split, Cs);
    __syncthreads();
    if constexpr (MODE != EPI_ENC && C::BN == 2 * kBN) {
      epilogue_pair<uint16_t, kFixRows, MODE, 256, 1>(Cs, LDC, meta, m0, n0, g);
    } else {
#pragma unroll 1
      for (int cb = 0; cb < C::BN / kBN; ++cb)
        epilogue<uint16_t, kFixRows, MODE, 256, 1>(Cs + cb * kBN, LDC, meta, m0, n0 + cb * kBN, g);
    }
  }
}

// 256x256 tiles, 8 waves of 128x64, two 64-deep ring slots (128 KB), one
// work-group per CU
using GemmBig = GemmCfg<256, 256, 2, 4, 2, 64>;
// 256x128 tiles, 8 waves of 64x64, three 64-deep ring slots (144 KB): about 15%
// less efficient per flop, but twice the tiles, for host-sized launches whose
// 256x256 tiles would leave most of a round idle
using GemmMid = GemmCfg<256, 128, 4, 2, 3, 64>;

// ------------------------------------------------------------------------- //
// fp32 kernel: 64x128 tile, BK 16, each thread 4 rows x 8 columns.
// ------------------------------------------------------------------------- //
constexpr int kBM32 = 64, kBK32 = 16;

template <int MODE>
__global__ __launch_bounds__(256, 2) void gemm_f32_kernel(GemmArgs g) {
  __shared__ __align__(16) float smem32[kBM32 * kLDC];  // 33,792 B; also holds A/B tiles
  __shared__ EpiRow meta32[kBM32];
  float *As = smem32;                     // [BK][BM+4]
  float *Bs = smem32 + kBK32 * (kBM32 + 4);  // [BK][BN+4]
  float *Cs = smem32;
  const int M = g.M_dev ? *g.M_dev : g.M_host;
  const int K = g.K, N = g.N;
  const int mt_n = (M + kBM32 - 1) / kBM32, nt_n = (N + kBN - 1) / kBN;
  const TileIter ti(mt_n * nt_n);
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const float *A = (const float *)g.A, *B = (const float *)g.B;

  for (int lt = ti.loc;; lt += ti.per_x) {
    const int tile = ti.tile(lt);
    if (tile < 0) break;
    const int mt = tile / nt_n, nt = tile - mt * nt_n;
    const int m0 = mt * kBM32, n0 = nt * kBN;
    load_row_meta<MODE, kBM32>(meta32, m0, M, g);
    float acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
    // loader mapping: A 64 rows x 16 k (one float4 per thread), B 128 rows x 16 k (two)
    const int ar = tid >> 2, ak = (tid & 3) * 4;
    const int am = m0 + ar;
    const float *pa = nullptr;
    if (am < M) pa = A + (size_t)(g.a_rows ? g.a_rows[am] : am) * K + ak;
    const float *pb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int n = n0 + ar + 64 * i;
      pb[i] = n < N ? B + (size_t)n * K + ak : nullptr;
    }
    for (int k0 = 0; k0 < K; k0 += kBK32) {
      float4 va = pa ? *reinterpret_cast<const float4 *>(pa + k0) : make_float4(0, 0, 0, 0);
      float4 vb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        vb[i] = pb[i] ? *reinterpret_cast<const float4 *>(pb[i] + k0) : make_float4(0, 0, 0, 0);
      __syncthreads();
      As[(ak + 0) * (kBM32 + 4) + ar] = va.x;
      As[(ak + 1) * (kBM32 + 4) + ar] = va.y;
      As[(ak + 2) * (kBM32 + 4) + ar] = va.z;
      As[(ak + 3) * (kBM32 + 4) + ar] = va.w;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int c = ar + 64 * i;
        Bs[(ak + 0) * (kBN + 4) + c] = vb[i].x;
        Bs[(ak + 1) * (kBN + 4) + c] = vb[i].y;
        Bs[(ak + 2) * (kBN + 4) + c] = vb[i].z;
        Bs[(ak + 3) * (kBN + 4) + c] = vb[i].w;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kBK32; ++k) {
        float av[4], bv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = As[k * (kBM32 + 4) + ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[j] = Bs[k * (kBN + 4) + tx + 16 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) Cs[(ty * 4 + i) * kLDC + tx + 16 * j] = acc[i][j];
    __syncthreads();
    epilogue<float, kBM32, MODE, 256, 4>(Cs, kLDC, meta32, m0, n0, g);
    __syncthreads();
  }
}

// Time of a launch of `tiles` tiles on `grid` work-groups in units of one tile's
// time: whole rounds, then the split last round (a piece plus the fix-up) or one
// more round.
inline float launch_cost(int tiles, int grid, int part_cap) {
  constexpr float kFixCost = 0.07f;
  const SplitPlan sp = split_plan(tiles, grid, part_cap);
  if (sp.split >= 2) return (float)(sp.full / grid) + 1.f / (float)sp.split + kFixCost;
  return (float)((tiles + grid - 1) / grid);
}

template <typename C>
hipError_t launch_gemm_cfg(GemmArgs g, hipStream_t s) {
  const bool bf = g.dtype == SRP_BF16;
  const int bm = bf ? C::BM : kBM32, bn = bf ? C::BN : kBN;
  const long tiles = (long)((g.M_cap + bm - 1) / bm) * ((g.N + bn - 1) / bn);
  if (tiles <= 0) return hipSuccess;
  // resident work-groups (256 CUs x work-groups per CU), a multiple of the 8 XCDs.
  // With room for partial tiles the grid stays whole, so that a launch of fewer
  // tiles than work-groups splits them along K (all of them form the last round).
  if (!bf || !g.part) g.part_cap = 0;
  const long resident = bf ? 256L * C::PER_CU : 512L;
  long grid = tiles < resident && g.part_cap == 0 ? tiles : resident;
  grid = (grid + 7) / 8 * 8;
  g.grid_main = (int)grid;
  const dim3 gr((unsigned)grid), bl(bf ? C::THREADS : 256);
  // fix-up: with M known here the split plan is known too (no launch without a
  // split); with M on the device, as many items as the plan can have for M_cap
  // rows. Up to 1024 work-groups stride over the items.
  long fix_items = 0;
  if (bf && g.part_cap > 0) {
    if (!g.M_dev) {
      const int mt_n = (g.M_host + C::BM - 1) / C::BM, nt_n = (g.N + C::BN - 1) / C::BN;
      const SplitPlan sp = split_plan(mt_n * nt_n, (int)grid, g.part_cap);
      fix_items = sp.split < 2 ? 0 : (long)sp.tail * (C::BM / kFixRows);
    } else {
      fix_items = (g.part_cap / 2 < tiles ? g.part_cap / 2 : tiles) * (C::BM / kFixRows);
    }
  }
  const long fix_tiles = fix_items;
  const dim3 fgr((unsigned)(fix_items > 0 ? (fix_items < 1024 ? fix_items : 1024) : 1));
#define SRP_GEMM_LAUNCH(M)                                                     \
  if (bf) {                                                                    \
    hipLaunchKernelGGL((gemm_bf16_kernel<M, C>), gr, bl, 0, s, g);             \
    if (fix_tiles > 0)                                                         \
      hipLaunchKernelGGL((gemm_fixup_kernel<M, C>), fgr, dim3(256), 0, s, g);  \
  } else {                                                                     \
    hipLaunchKernelGGL(gemm_f32_kernel<M>, gr, bl, 0, s, g);                   \
  }
  switch (g.mode) {
    case EPI_KV: SRP_GEMM_LAUNCH(EPI_KV); break;
    case EPI_Q: SRP_GEMM_LAUNCH(EPI_Q); break;
    case EPI_V: SRP_GEMM_LAUNCH(EPI_V); break;
    case EPI_QK: SRP_GEMM_LAUNCH(EPI_QK); break;
    default: SRP_GEMM_LAUNCH(EPI_ENC); break;
  }
#undef SRP_GEMM_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t s) {
  // bf16 with M known on the host: 256x128 tiles when the estimate says they end
  // the launch at least 10% sooner (a 256x128 tile takes about 0.59 of a 256x256
  // one); M on the device (sized for M_cap) keeps 256x256.
  if (g.dtype == SRP_BF16 && !g.M_dev && g.part) {
    const int M = g.M_host;
    const long big = (long)((M + GemmBig::BM - 1) / GemmBig::BM) * ((g.N + GemmBig::BN - 1) / GemmBig::BN);
    const long mid = (long)((M + GemmMid::BM - 1) / GemmMid::BM) * ((g.N + GemmMid::BN - 1) / GemmMid::BN);
    if (big > 0 && big < (1L << 30) &&
        0.59f * launch_cost((int)mid, 256, g.part_cap) < 0.9f * launch_cost((int)big, 256, g.part_cap))
      return launch_gemm_cfg<GemmMid>(g, s);
  }
  return launch_gemm_cfg<GemmBig>(g, s);
}

}  // namespace srp
