// Gathered-query causal GQA flash attention over the fused cache (gfx950).
//
// bf16: a work-group is (tile of selected rows of one request, KV head g) and
// eight waves, two per SIMD. Its 256 MFMA columns are (query, head) pairs of the
// group, query-major: column c is query c / G, head c % G, so every K/V tile
// staged in LDS serves all G heads that read it and the waves stay balanced for
// any G <= 8 (G = 5 packs 51 queries x 5 heads). Each wave computes, for its 32
// columns, S^T = K Q^T and O^T = V^T P^T with v_mfma_f32_32x32x16_bf16: a lane
// holds one column, so the online-softmax max needs one exchange between lanes
// l and l+32 and the rescale of O is per lane. The probabilities are reused in
// registers as the B operand of the PV product; V is staged in LDS transposed,
// with the keys of every 16-key group stored in the order that operand reads
// them, so each V fragment is one 16-byte LDS read. Causality is by row:
// positions rise strictly inside a request.
#include <type_traits>

#include "kernels.hpp"

namespace srp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Calls f(integral_constant<int, i>) for i = 0..N-1, so array indices inside f
// are compile-time constants (register arrays stay in registers).
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

constexpr int kBK = kAttnBK;     // keys per LDS stage
constexpr int kAW = 8;           // waves per work-group (two per SIMD)
constexpr int kACols = 32 * kAW; // (query, head) columns per work-group

// max of x over lanes l and l^32 (v_permlane32_swap: no LDS round trip)
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Software pipelined: each wave overlaps the score MFMAs of key tile j+1 with the
// exponentials of tile j, and the PV MFMAs of tile j with the mask and max of
// tile j+1, so its own VALU work runs under its own matrix work. Waves 4-7 run
// half an iteration behind waves 0-3 (one barrier per tile, at a different point
// of the iteration for each group), so the two waves on a SIMD are in opposite
// halves. A five-slot ring gives each tile's copy two iterations to land.
template <int D>
__global__ __launch_bounds__(64 * kAW, 1) void attn_bf16_kernel(AttnArgs a) {
  // K tile: 64 rows of D bf16 (D*2 bytes), 16-byte chunk c of row r stored at
  // c ^ (r % KCH). V^T tile: D rows of 64 keys (128 bytes), chunk c of row r
  // stored at c ^ ((r / 2) % 8). A 16-byte LDS read serves 16 lanes (64 banks)
  // per cycle; the fragment reads put 16 consecutive rows in those lanes, and
  // both layouts give them 16 different bank groups.
  constexpr int KT = kBK * D * 2, VT = D * kBK * 2, STAGE = KT + VT;
  constexpr int KCH = D / 8;
  constexpr int KROWS = 64 / KCH;
  constexpr int KJ = kBK / KROWS / kAW;
  constexpr int VJ = D / 8 / kAW;
  constexpr int LOADS = KJ + VJ;
  constexpr int NS = D / 16;
  constexpr int PFD = 3;  // LDS fragment reads issued this many MFMAs ahead
  static_assert(KJ >= 1 && VJ >= 1, "every wave copies K and V^T rows");
  constexpr int NSL = 5;  // ring slots
  // the ring slots as separate LDS objects: every access below names its slot at
  // compile time
  __shared__ __align__(16) char st0[STAGE];
  __shared__ __align__(16) char st1[STAGE];
  __shared__ __align__(16) char st2[STAGE];
  __shared__ __align__(16) char st3[STAGE];
  __shared__ __align__(16) char st4[STAGE];
  auto slot_ptr = [&](auto I) __attribute__((always_inline)) -> char * {
    if constexpr (decltype(I)::value == 0) return st0;
    else if constexpr (decltype(I)::value == 1) return st1;
    else if constexpr (decltype(I)::value == 2) return st2;
    else if constexpr (decltype(I)::value == 3) return st3;
    else return st4;
  };

  const int n_tiles = *a.n_tiles;
  const int slot = blockIdx.x / a.nkv, g = blockIdx.x - slot * a.nkv;
  if (slot >= n_tiles) return;
  const int G = a.nh / a.nkv;
  const int q0 = a.tiles[3 * slot], nq = a.tiles[3 * slot + 1], r = a.tiles[3 * slot + 2];
  if (nq <= 0) return;  // the empty second half of a one-row tile
  // key tiles are aligned to 64 rows (the V^T key order repeats every 16 rows
  // and the copies stay 128-byte aligned); rows of the first tile before the
  // request's first row are masked
  const int key_start = a.req_offsets[r];
  const int key_base = key_start & ~(kBK - 1);
  const int last_row = a.sel_idx[q0 + nq - 1];
  const int key_end = last_row + 1;
  const int nblk = (key_end - key_base + kBK - 1) / kBK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = lane & 31, gph = lane >> 5;
  const int col = 32 * w + qi;
  const int qq = col / G, hh = col - qq * G;
  const bool cvalid = qq < nq;
  const int qrow = a.sel_idx[q0 + (cvalid ? qq : nq - 1)];
  // the wave's first and last query rows (uniform): tiles that end after the
  // first are masked, tiles that start after the last are skipped. A wave with
  // no query columns skips every tile but still copies and meets the barriers.
  const int wq_lo = (32 * w) / G, wq_hi = min(nq - 1, (32 * w + 31) / G);
  const bool wactive = wq_lo < nq;
  const int w_first = wactive ? a.sel_idx[q0 + wq_lo] : key_end;
  const int w_last = wactive ? a.sel_idx[q0 + wq_hi] : key_start - 1;
  // key tiles this wave computes (those starting at or before its last query)
  const int nact = wactive ? min(nblk, (w_last - key_base) / kBK + 1) : 0;
  const size_t row_bytes = (size_t)a.nkv * D * 2;
  const char *Kg = (const char *)a.k_cache + (size_t)g * D * 2;
  const char *Vg = (const char *)a.vt + (size_t)g * D * a.vt_stride * 2;
  const size_t vrow_bytes = (size_t)a.vt_stride * 2;

  // Wave w copies K rows KROWS*i.. (i = w + 8j) and V^T rows 8i.. per tile; each
  // lane's source offset inside a copy is a constant (the swizzle term only
  // depends on the lane for these row groups). Rows past key_end are clamped to
  // the last valid row; such keys come after every query of the tile and are masked.
  const int k_lrow = lane / KCH, k_logical = (lane % KCH) ^ ((KROWS * w + k_lrow) & (KCH - 1));
  const uint32_t k_chunk_off = (uint32_t)(k_logical * 16), row_bytes32 = (uint32_t)row_bytes;
  const int v_lrow = lane >> 3, v_logical = (lane & 7) ^ (((8 * w + v_lrow) >> 1) & 7);
  const uint32_t v_lane_off = (uint32_t)(v_lrow * vrow_bytes + v_logical * 16);
  auto issue = [&](auto SLOT, int blk) __attribute__((always_inline)) {
    const int kb = key_base + blk * kBK;
    char *st = slot_ptr(SLOT);
    static_for<KJ>([&](auto J) __attribute__((always_inline)) {
      const int i = w + kAW * decltype(J)::value;
      // lane row min(kb + KROWS i + k_lrow, key_end - 1) as a wave-uniform first
      // row plus a small per-lane step (24-bit multiply, no 64-bit lane math)
      const int r0 = min(kb + KROWS * i, key_end - 1);
      const uint32_t lo = __umul24((uint32_t)min(k_lrow, key_end - 1 - r0), row_bytes32) + k_chunk_off;
      dma16(Kg + (size_t)r0 * row_bytes + lo, st + i * 1024);
    });
    static_for<VJ>([&](auto J) __attribute__((always_inline)) {
      const int i = w + kAW * decltype(J)::value;
      dma16(Vg + (size_t)(8 * i) * vrow_bytes + (size_t)kb * 2 + v_lane_off, st + KT + i * 1024);
    });
  };

  // Q fragments (B operand of S^T = K Q^T): lane holds its column's query row,
  // d range ks*16 + gph*8 .. +8, in registers for the whole tile
  u32x4 qf[NS];
  {
    const uint16_t *qp =
        (const uint16_t *)a.q + ((size_t)(q0 + (cvalid ? qq : 0)) * a.nh + g * G + hh) * D + gph * 8;
#pragma unroll
    for (int ks = 0; ks < NS; ++ks)
      qf[ks] = cvalid ? *reinterpret_cast<const u32x4 *>(qp + ks * 16) : u32x4{0, 0, 0, 0};
  }
  // the Q loads complete before the first tile copy is issued: the copies are
  // invisible to the compiler's wait counting, which would otherwise wait for
  // every outstanding load (the whole ring) at each use of Q
  wait_vmcnt<0>();
  floatx16 acc[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
  // Scores are in base-2 units (queries carry log2(e)/sqrt(d)). The score chains
  // start at -m, so they come out of the MFMA already relative to the reference
  // max m, which is raised only when a tile's max exceeds it by more than 8:
  // probabilities stay below 2^8 and rescales are rare. The check follows the
  // exponentials instead of a max before them: a probability of at least 2^8 makes
  // its lane's sum over the tile at least 256, and only then (rarely) is the exact
  // max taken and the tile redone. l is this lane's share of the row sum (its keys
  // of each 16-key step); the two lanes of a column are added at the end.
  float m = 0.f, l = 0.f;
  floatx16 cneg;  // -m in every element: the first accumulator of each score chain
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  uint32_t koff[NS];
#pragma unroll
  for (int ks = 0; ks < NS; ++ks) koff[ks] = qi * (D * 2) + (((2 * ks + gph) ^ (qi & (KCH - 1))) * 16);
  uint32_t voff[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) voff[c] = KT + qi * 128 + (((2 * c + gph) ^ ((qi >> 1) & 7)) * 16);
  // the same lane offsets 64 KB further on: fragment reads of the slots that lie
  // beyond the 16-bit immediate offset of an LDS read start from these registers
  uint32_t koff_hi[NS], voff_hi[4];
#pragma unroll
  for (int ks = 0; ks < NS; ++ks) koff_hi[ks] = koff[ks] + 65536u;
#pragma unroll
  for (int c = 0; c < 4; ++c) voff_hi[c] = voff[c] + 65536u;

  // S^T of the first tile (both 32-key halves) into s, starting from c0; K
  // fragments two steps ahead, kept in that order by the scheduling barriers
  auto qk = [&](auto SLOT, floatx16 (&s)[2], float c0) __attribute__((always_inline)) {
    const char *St = slot_ptr(SLOT);
    auto kfrag = [&](int t) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8 *>(St + koff[t % NS] + (t / NS) * 32 * (D * 2));
    };
#pragma unroll
    for (int e = 0; e < 16; ++e) { s[0][e] = c0; s[1][e] = c0; }
    bf16x8 kf[3];
    kf[0] = kfrag(0);
    kf[1] = kfrag(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2 * NS; ++t) {
      if (t + 2 < 2 * NS) kf[(t + 2) % 3] = kfrag(t + 2);
      const bf16x8 q8 = __builtin_bit_cast(bf16x8, qf[t % NS]);
      s[t / NS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t % 3], q8, s[t / NS], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // causal / request mask of the tile at kb, then the column max
  auto mask_max = [&](floatx16 (&s)[2], int kb) __attribute__((always_inline)) {
    if (kb < key_start || kb + kBK - 1 > w_first) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int krow = kb + hb * 32 + (e >> 2) * 8 + gph * 4 + (e & 3);
          if (krow > qrow || krow < key_start) s[hb][e] = -INFINITY;
        }
    }
    float x = __builtin_fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int e = 2; e < 16; e += 2) x = __builtin_fmaxf(__builtin_fmaxf(x, s[0][e]), s[0][e + 1]);
#pragma unroll
    for (int e = 0; e < 16; e += 2) x = __builtin_fmaxf(__builtin_fmaxf(x, s[1][e]), s[1][e + 1]);
    return pair_max(x);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  floatx16 sa[2], sb[2];
  // tiles 0-3 in flight; 0 and 1 are read before the first barrier of the loop
  issue(I0{}, 0);
  if (nblk > 1) issue(I1{}, 1);
  if (nblk > 2) issue(I2{}, 2);
  if (nblk > 3) issue(I3{}, 3);
  if (nblk > 3) wait_vmcnt<2 * LOADS>();
  else if (nblk > 2) wait_vmcnt<LOADS>();
  else wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  if (nact > 0) {
    // the first tile sets the reference max (it holds the request's first row,
    // which every query sees, so the max is finite)
    qk(I0{}, sa, 0.f);
    const float mx = mask_max(sa, key_base);
    m = mx;
#pragma unroll
    for (int e = 0; e < 16; ++e) cneg[e] = -m;
#pragma unroll
    for (int e = 0; e < 16; ++e) { sa[0][e] -= mx; sa[1][e] -= mx; }
  }
  // One step of the overlapped part of iteration j: the MFMA of step t, then
  // VALU work that does not depend on it, with fragment reads PFD steps ahead;
  // the scheduling barriers keep that order (the compiler would otherwise move
  // every LDS read to the top and run out of registers).
  // Part 1: the score MFMAs of tile j+1 (chain 0 for keys 0-31, chain 1 for keys
  // 32-63, taken in turn so neither waits on its own previous MFMA) with the
  // probabilities of tile j: step t exponentiates elements
  // 2(t%4), 2(t%4)+1 of k-step c = t/4 (half c/2, elements 8(c%2)+...).
  auto part1 = [&](auto NSLOT, floatx16 (&cur)[2], floatx16 (&nxt)[2], u32x4 (&pw)[4], float &lt)
      __attribute__((always_inline)) {
    const char *St = slot_ptr(NSLOT);
    auto kfrag = [&](int t) __attribute__((always_inline)) {
      const uint32_t so = (uint32_t)(uintptr_t)(lds_void *)St;
      const uint32_t a = so >= 65536u ? koff_hi[t >> 1] + (so - 65536u) : koff[t >> 1] + so;
      return *(const __attribute__((address_space(3))) bf16x8 *)(uintptr_t)(a + (t & 1) * 32 * (D * 2));
    };
    bf16x8 kf[PFD + 1];
#pragma unroll
    for (int t = 0; t < PFD; ++t) kf[t] = kfrag(t);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2 * NS; ++t) {
      if (t + PFD < 2 * NS) kf[(t + PFD) % (PFD + 1)] = kfrag(t + PFD);
      const bf16x8 q8 = __builtin_bit_cast(bf16x8, qf[t >> 1]);
      // each chain starts from -m held in registers (no per-tile initialisation)
      nxt[t & 1] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[t % (PFD + 1)], q8, t < 2 ? cneg : nxt[t & 1], 0, 0, 0);
      // VALU share of this step (16 steps of D = 128; D = 64 has 8, two shares each)
#pragma unroll
      for (int u = 0; u < 16 / (2 * NS); ++u) {
        const int v = t * (16 / (2 * NS)) + u;  // 0..15
        const int c = v / 4, jj = 2 * (v % 4);
        const bf16x2 pr = {(__bf16)__builtin_amdgcn_exp2f(cur[c / 2][(c % 2) * 8 + jj]),
                           (__bf16)__builtin_amdgcn_exp2f(cur[c / 2][(c % 2) * 8 + jj + 1])};
        uint32_t word = __builtin_bit_cast(uint32_t, pr);
        lt = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lt, false);
        // the empty asm pins the work to this step (it would otherwise sink to
        // its first use, the PV MFMAs)
        asm volatile("" : "+v"(word), "+v"(lt));
        pw[c][v % 4] = word;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // After the exponentials of tile j (scores cur): when some lane's sum over the
  // tile reached 256, the tile's exact column max decides a rescale as in the
  // lazy scheme (raise m where it exceeds 8; O, l and the next tile's scores follow)
  // and the tile's probabilities are formed again. Wave-uniform and rare.
  auto check_tile = [&](floatx16 (&cur)[2], floatx16 (&nxt)[2], u32x4 (&pw)[4], float &lt)
      __attribute__((always_inline)) {
    if (__any(lt >= 256.f)) {
      float x = __builtin_fmaxf(cur[0][0], cur[0][1]);
#pragma unroll
      for (int e = 2; e < 16; e += 2) x = __builtin_fmaxf(__builtin_fmaxf(x, cur[0][e]), cur[0][e + 1]);
#pragma unroll
      for (int e = 0; e < 16; e += 2) x = __builtin_fmaxf(__builtin_fmaxf(x, cur[1][e]), cur[1][e + 1]);
      x = pair_max(x);
      const bool up = x > 8.f;
      if (__any(up)) {
        const float dlt = up ? x : 0.f;
        const float alpha = __builtin_amdgcn_exp2f(-dlt);
        m += dlt;
#pragma unroll
        for (int e = 0; e < 16; ++e) cneg[e] = -m;
        l *= alpha;
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[b][e] *= alpha;
#pragma unroll
        for (int e = 0; e < 16; ++e) { nxt[0][e] -= dlt; nxt[1][e] -= dlt; }
        lt = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int c = v / 4, jj = 2 * (v % 4);
          const bf16x2 pr = {(__bf16)__builtin_amdgcn_exp2f(cur[c / 2][(c % 2) * 8 + jj] - dlt),
                             (__bf16)__builtin_amdgcn_exp2f(cur[c / 2][(c % 2) * 8 + jj + 1] - dlt)};
          lt = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lt, false);
          pw[c][v % 4] = __builtin_bit_cast(uint32_t, pr);
        }
      }
    }
    l += lt;
  };
  // Part 2: the PV MFMAs of tile j, with the mask of tile j+1 when it needs one
  // (its VALU work now lies in part 1, which the other wave of the SIMD runs meanwhile)
  auto part2 = [&](auto SLOT, floatx16 (&nxt)[2], const u32x4 (&pw)[4], int kb_next)
      __attribute__((always_inline)) {
    const char *St = slot_ptr(SLOT);
    auto vfrag = [&](int t) __attribute__((always_inline)) {
      const uint32_t so = (uint32_t)(uintptr_t)(lds_void *)St;
      const uint32_t a = so >= 65536u ? voff_hi[t / (D / 32)] + (so - 65536u) : voff[t / (D / 32)] + so;
      return *(const __attribute__((address_space(3))) bf16x8 *)(uintptr_t)(a + (t % (D / 32)) * 32 * 128);
    };
    if (kb_next < key_start || kb_next + kBK - 1 > w_first) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int krow = kb_next + hb * 32 + (e >> 2) * 8 + gph * 4 + (e & 3);
          if (krow > qrow || krow < key_start) nxt[hb][e] = -INFINITY;
        }
    }
    constexpr int NPV = 4 * (D / 32);  // PV MFMAs per tile
    bf16x8 vf[PFD + 1];
#pragma unroll
    for (int t = 0; t < PFD; ++t) vf[t] = vfrag(t);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NPV; ++t) {
      if (t + PFD < NPV) vf[(t + PFD) % (PFD + 1)] = vfrag(t + PFD);
      const int b = t % (D / 32);
      acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[t % (PFD + 1)], __builtin_bit_cast(bf16x8, pw[t / (D / 32)]),
                                                       acc[b], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // iteration j: tile j's scores are in `cur`, tile j+1's go to `nxt`. A wave's
  // last tile runs the same code (its score MFMAs read a stale slot and their
  // results are dropped): one straight-line body keeps the compiler from
  // merging the two paths' exponentials ahead of the MFMAs.
  // Barrier b_j ends iteration j (for waves 0-3; waves 4-7 meet it between
  // their two parts); before it every wave waits for its copies of tile j+2,
  // after it tile j+4 is issued into the slot of tile j-1, which no wave reads
  // after b_j.
  auto barrier_after = [&](int j) __attribute__((always_inline)) {
    if (j + 3 < nblk) wait_vmcnt<LOADS>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  };
  const bool lead = w < kAW / 2;
  auto iter = [&](auto SLOT, int j, floatx16 (&cur)[2], floatx16 (&nxt)[2]) __attribute__((always_inline)) {
    constexpr int sl = decltype(SLOT)::value;
    using NEXT = std::integral_constant<int, (sl + 1) % NSL>;
    using FREE3 = std::integral_constant<int, (sl + 3) % NSL>;
    using FREE4 = std::integral_constant<int, (sl + 4) % NSL>;
    // Waves 4-7 run half an iteration behind: their barrier b_j falls between
    // the score MFMAs of tile j+1 and the PV MFMAs of tile j, so on each SIMD one
    // wave's exponentials overlap the other's PV product. They issue tile j+4
    // right after b_j; waves 0-3 issue it at the start of iteration j+1.
    const bool second = !lead;
    if (!second && j >= 1 && j + 3 < nblk) issue(FREE3{}, j + 3);
    u32x4 pw[4];
    if (j < nact) {
      float lt = 0.f;
      part1(NEXT{}, cur, nxt, pw, lt);
      check_tile(cur, nxt, pw, lt);
    }
    if (second && j + 1 < nblk) {
      barrier_after(j);
      if (j + 4 < nblk) issue(FREE4{}, j + 4);
    }
    if (j < nact) part2(SLOT, nxt, pw, key_base + (j + 1) * kBK);
    if (!second && j + 1 < nblk) barrier_after(j);
  };
  // unrolled by ten so slots and score buffers are both constants
  for (int j0 = 0; j0 < nblk; j0 += 10) {
    iter(I0{}, j0, sa, sb);
    if (j0 + 1 < nblk) iter(I1{}, j0 + 1, sb, sa);
    if (j0 + 2 < nblk) iter(I2{}, j0 + 2, sa, sb);
    if (j0 + 3 < nblk) iter(I3{}, j0 + 3, sb, sa);
    if (j0 + 4 < nblk) iter(I4{}, j0 + 4, sa, sb);
    if (j0 + 5 < nblk) iter(I0{}, j0 + 5, sb, sa);
    if (j0 + 6 < nblk) iter(I1{}, j0 + 6, sa, sb);
    if (j0 + 7 < nblk) iter(I2{}, j0 + 7, sb, sa);
    if (j0 + 8 < nblk) iter(I3{}, j0 + 8, sa, sb);
    if (j0 + 9 < nblk) iter(I4{}, j0 + 9, sb, sa);
  }

  const float lt = pair_sum(l);
  if (cvalid) {
    const float inv = 1.f / lt;
    uint16_t *op = (uint16_t *)a.out + ((size_t)(q0 + qq) * a.nh + g * G + hh) * D;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (__bf16)(acc[b][e4 * 4 + i] * inv);
        *reinterpret_cast<bf16x4 *>(op + b * 32 + e4 * 8 + gph * 4) = v;
      }
  }
}

// fp32 variant: one wave per head, one query at a time, one key per lane.
template <int D>
__global__ __launch_bounds__(512) void attn_f32_kernel(AttnArgs a) {
  const int n_tiles = *a.n_tiles;
  const int slot = blockIdx.x / a.nkv, g = blockIdx.x - slot * a.nkv;
  if (slot >= n_tiles) return;
  const int G = a.nh / a.nkv;
  const int q0 = a.tiles[3 * slot], nq = a.tiles[3 * slot + 1], r = a.tiles[3 * slot + 2];
  const int key_start = a.req_offsets[r];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int h = g * G + w;
  const size_t kvd = (size_t)a.nkv * D;
  const float *K = (const float *)a.k_cache + g * D;
  const float *V = (const float *)a.v_cache + g * D;
  constexpr int C = D / 64;
  const float scale = 1.f / sqrtf((float)D);
  for (int qi = 0; qi < nq; ++qi) {
    const int row = a.sel_idx[q0 + qi];
    const float *q = (const float *)a.q + ((size_t)(q0 + qi) * a.nh + h) * D;
    float m = -INFINITY, l = 0.f, o[C];
#pragma unroll
    for (int c = 0; c < C; ++c) o[c] = 0.f;
    for (int kb = key_start; kb <= row; kb += 64) {
      const int key = kb + lane;
      float s = -INFINITY;
      if (key <= row) {
        const float *kr = K + (size_t)key * kvd;
        float acc = 0.f;
        for (int i = 0; i < D; ++i) acc = fmaf(q[i], kr[i], acc);
        s = acc * scale;
      }
      float mx = s;
      for (int o2 = 32; o2 > 0; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2, 64));
      const float m_new = fmaxf(m, mx);
      const float alpha = expf(m - m_new);
      const float p = key <= row ? expf(s - m_new) : 0.f;
      float ps = p;
      for (int o2 = 32; o2 > 0; o2 >>= 1) ps += __shfl_xor(ps, o2, 64);
      l = l * alpha + ps;
      m = m_new;
#pragma unroll
      for (int c = 0; c < C; ++c) o[c] *= alpha;
      const int nk = row - kb + 1 < 64 ? row - kb + 1 : 64;
      for (int kk = 0; kk < nk; ++kk) {
        const float pk = __shfl(p, kk, 64);
        const float *vr = V + (size_t)(kb + kk) * kvd;
#pragma unroll
        for (int c = 0; c < C; ++c) o[c] = fmaf(pk, vr[lane + 64 * c], o[c]);
      }
    }
    float *op = (float *)a.out + ((size_t)(q0 + qi) * a.nh + h) * D;
#pragma unroll
    for (int c = 0; c < C; ++c) op[lane + 64 * c] = o[c] / l;
  }
}

int attn_tile_rows(int dtype, int nh, int nkv) {
  return dtype == SRP_BF16 ? kACols / (nh / nkv) : 32;
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t s) {
  const int G = a.nh / a.nkv;
  const dim3 grid((unsigned)(a.max_tiles * a.nkv));
  if (a.dtype == SRP_BF16) {
    if (a.d == 128) hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(64 * kAW), 0, s, a);
    else hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(64 * kAW), 0, s, a);
  } else {
    const dim3 block((unsigned)(64 * G));
    if (a.d == 128) hipLaunchKernelGGL(attn_f32_kernel<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace srp
