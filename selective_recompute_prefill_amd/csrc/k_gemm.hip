// Gathered projection GEMMs with the layer's epilogues (gfx950).
//
// C = A_gathered * W^T: A rows are token rows picked by an index list (the
// candidates and fresh rows for K/V, the selected rows for Q), W rows are output
// features. The bf16 kernel uses v_mfma_f32_32x32x16_bf16 with fp32 accumulation;
// the fp32 kernel is a plain FMA tiling for fp32 workloads. Both stage the
// accumulator tile in LDS and run the same epilogue, which works on whole heads so
// that each rotation pair (i, i + d/2) sits in one thread.
#include "kernels.hpp"

namespace srp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kBN = 128;

// ------------------------------------------------------------------------- //
// epilogue
// ------------------------------------------------------------------------- //
template <typename T, int BM, int MODE>
__device__ __forceinline__ void epilogue(const float *Cs, int ldc, int m0, int n0, int M,
                                         const GemmArgs &g) {
  const int d = g.d, half = d >> 1;
  const int tpu = d >> 3;          // threads per head unit (4 pairs each)
  const int kvd = g.nkv * d;
  for (int it = threadIdx.x; it < BM * 16; it += blockDim.x) {
    const int r = it >> 4, qq = it & 15;
    const int u = qq / tpu, t = qq - u * tpu;
    const int m = m0 + r;
    const int nu = n0 + u * d;
    const bool valid = (m < M) && (nu < g.N);
    const int i0 = t * 4;
    float a[4], b[4];
    const float *src = Cs + r * ldc + u * d;
#pragma unroll
    for (int k = 0; k < 4; ++k) { a[k] = src[i0 + k]; b[k] = src[half + i0 + k]; }
    float part_sum = 0.f;
    int slot = -1;
    if (valid) {
      const int row = (MODE != EPI_ENC && g.a_rows) ? g.a_rows[m] : m;
      if (MODE == EPI_Q) {
        const int h = nu / d;
        rope4(a, b, g.rope, g.positions[row], i0);
#pragma unroll
        for (int k = 0; k < 4; ++k) { a[k] *= g.q_scale; b[k] *= g.q_scale; }
        T *q = (T *)g.q_out + (size_t)m * g.nh * d + h * d;
        st4(q + i0, a);
        st4(q + half + i0, b);
      } else {
        const int part = nu >= kvd;
        const int gh = (nu - part * kvd) / d;
        if (part == 0) rope4(a, b, g.rope, g.positions[row], i0);
        if (MODE == EPI_ENC) {
          T *o = (T *)(part ? g.v_cache : g.k_cache) + (size_t)m * kvd + gh * d;
          st4(o + i0, a);
          st4(o + half + i0, b);
        } else {
          T *f = (T *)g.fresh + (size_t)m * 2 * kvd + part * kvd + gh * d;
          st4(f + i0, a);
          st4(f + half + i0, b);
          const int delta = g.row_delta[row];
          slot = part * g.nkv + gh;
          if (delta != kFresh) {
            T *c = (T *)(part ? g.v_cache : g.k_cache) + (size_t)row * kvd + gh * d;
            float ca[4], cb[4];
            ld4(c + i0, ca);
            ld4(c + half + i0, cb);
            if (part == 0) {
              // positional recovery of the cached key, kept in fp32 for the
              // deviation and written back to the cache
              rope4(ca, cb, g.rope, delta, i0);
              st4(c + i0, ca);
              st4(c + half + i0, cb);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              float x = a[k] - ca[k], y = b[k] - cb[k];
              part_sum += x * x + y * y;
            }
          }
        }
      }
    }
    if (MODE == EPI_KV) {
      // fixed-order reduction over the head's tpu lanes (aligned groups)
      for (int o = 1; o < tpu; o <<= 1) part_sum += __shfl_xor(part_sum, o, 64);
      if (valid && t == 0) g.dev_part[(size_t)m * 2 * g.nkv + slot] = part_sum;
    }
  }
}

// ------------------------------------------------------------------------- //
// tile scheduling: persistent loop, each XCD (blockIdx % 8) walks a contiguous
// range of row-major tiles so the row block of A it reads stays in its L2
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
// bf16 MFMA kernel: 128x128 tile, BK 64, 4 waves (2x2), wave tile 64x64 made of
// 2x2 blocks of 32x32x16 MFMA. Operand tiles stream into an LDS ring with
// direct-to-LDS copies (no staging registers): copy i of a tile moves rows
// 8i..8i+7 (128 bytes each). Chunk c of row r is stored at c ^ ((r / 2) % 8):
// a 16-byte LDS read serves 16 lanes (64 banks) per cycle, and the fragment
// reads put 16 consecutive rows in those lanes, which this layout spreads over
// 16 different bank groups.
// ------------------------------------------------------------------------- //
#ifndef SRP_GEMM_STAGES
#define SRP_GEMM_STAGES 2
#endif
constexpr int kBM16 = 128, kBK16 = 64;
constexpr int kGStages = SRP_GEMM_STAGES;
constexpr int kGTile = kBM16 * kBK16 * 2;  // bytes of one operand tile (16 KB)
constexpr int kGStage = 2 * kGTile;         // A tile then B tile
constexpr int kLDC = kBN + 4;
constexpr int kGSmem = kGStages * kGStage > kBM16 * kLDC * 4 ? kGStages * kGStage : kBM16 * kLDC * 4;

template <int MODE>
__global__ __launch_bounds__(256, kGStages >= 3 ? 1 : 2) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __align__(16) char smem[kGSmem];
  float *Cs = reinterpret_cast<float *>(smem);  // epilogue staging, 128 x 132 fp32

  const int M = g.M_dev ? *g.M_dev : g.M_host;
  const int K = g.K, N = g.N;
  const int mt_n = (M + kBM16 - 1) / kBM16, nt_n = (N + kBN - 1) / kBN;
  const TileIter ti(mt_n * nt_n);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const char *A = (const char *)g.A, *B = (const char *)g.B;
  const int KT = K / kBK16;
  const size_t rowb = (size_t)K * 2;
  // copy layout: lane covers row 8i + lrow, physical chunk lane%8 <- logical
  // chunk lchunk; for the rows i = w + 4j of this wave the swizzle term is a
  // per-lane constant
  const int lrow = lane >> 3, lchunk = (lane & 7) ^ (((8 * w + lrow) >> 1) & 7);

  for (int lt = ti.loc;; lt += ti.per_x) {
    const int tile = ti.tile(lt);
    if (tile < 0) break;
    const int mt = tile / nt_n, nt = tile - mt * nt_n;
    const int m0 = mt * kBM16, n0 = nt * kBN;

    // wave w copies A rows and B rows of copies i = w + 4j; rows past M or N
    // read a valid row (their results are never stored)
    const char *pa[4], *pb[4];
    const int row0 = g.a_rows ? g.a_rows[m0] : m0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 8 * (w + 4 * j) + lrow;
      const int m = m0 + r, n = n0 + r;
      const int row = m < M ? (g.a_rows ? g.a_rows[m] : m) : row0;
      pa[j] = A + (size_t)row * rowb + lchunk * 16;
      pb[j] = B + (size_t)(n < N ? n : N - 1) * rowb + lchunk * 16;
    }
    auto issue = [&](int kt) __attribute__((always_inline)) {
      char *st = smem + (kt % kGStages) * kGStage;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        dma16(pa[j] + (size_t)kt * 128, st + (w + 4 * j) * 1024);
        dma16(pb[j] + (size_t)kt * 128, st + kGTile + (w + 4 * j) * 1024);
      }
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

#pragma unroll
    for (int p = 0; p < kGStages - 1; ++p)
      if (p < KT) issue(p);
    const int fr = lane & 31, fk = lane >> 5;
    for (int kt = 0; kt < KT; ++kt) {
      // this tile's copies are done once at most the later prefetched tiles'
      // copies (8 per tile per wave) are outstanding
      const int later = min(KT - 1 - kt, kGStages - 2);
      if (later >= 2) wait_vmcnt<16>();
      else if (later == 1) wait_vmcnt<8>();
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      // the slot of tile kt+S-1 was last read in iteration kt-1
      if (kt + kGStages - 1 < KT) issue(kt + kGStages - 1);
      const char *as = smem + (kt % kGStages) * kGStage, *bs = as + kGTile;
#pragma unroll
      for (int ks = 0; ks < kBK16 / 16; ++ks) {
        bf16x8 af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = wm * 64 + i * 32 + fr;
          af[i] = *reinterpret_cast<const bf16x8 *>(as + r * 128 + (((2 * ks + fk) ^ ((r >> 1) & 7)) * 16));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = wn * 64 + j * 32 + fr;
          bfr[j] = *reinterpret_cast<const bf16x8 *>(bs + r * 128 + (((2 * ks + fk) ^ ((r >> 1) & 7)) * 16));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave is done with the ring before it becomes Cs
    // stage the accumulators: D[row][col], row = 8*(e/4) + 4*(lane/32) + e%4
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = wm * 64 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
          const int col = wn * 64 + j * 32 + (lane & 31);
          Cs[row * kLDC + col] = acc[i][j][e];
        }
    __syncthreads();
    epilogue<uint16_t, kBM16, MODE>(Cs, kLDC, m0, n0, M, g);
    __syncthreads();
  }
}

// ------------------------------------------------------------------------- //
// fp32 kernel: 64x128 tile, BK 16, each thread 4 rows x 8 columns.
// ------------------------------------------------------------------------- //
constexpr int kBM32 = 64, kBK32 = 16;

template <int MODE>
__global__ __launch_bounds__(256, 2) void gemm_f32_kernel(GemmArgs g) {
  __shared__ __align__(16) float smem32[kBM32 * kLDC];  // 33,792 B; also holds A/B tiles
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
    epilogue<float, kBM32, MODE>(Cs, kLDC, m0, n0, M, g);
    __syncthreads();
  }
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t s) {
  const int bm = g.dtype == SRP_BF16 ? kBM16 : kBM32;
  const long tiles = (long)((g.M_cap + bm - 1) / bm) * ((g.N + kBN - 1) / kBN);
  if (tiles <= 0) return hipSuccess;
  // resident work-groups (256 CUs x work-groups per CU), a multiple of the 8 XCDs
  const long resident = g.dtype == SRP_BF16 ? 256L * (kGStages >= 3 ? 1 : 2) : 512L;
  long grid = tiles < resident ? tiles : resident;
  grid = (grid + 7) / 8 * 8;
  const dim3 gr((unsigned)grid), bl(256);
#define SRP_GEMM_LAUNCH(M)                                               \
  if (g.dtype == SRP_BF16)                                               \
    hipLaunchKernelGGL(gemm_bf16_kernel<M>, gr, bl, 0, s, g);            \
  else                                                                   \
    hipLaunchKernelGGL(gemm_f32_kernel<M>, gr, bl, 0, s, g);
  switch (g.mode) {
    case EPI_KV: SRP_GEMM_LAUNCH(EPI_KV); break;
    case EPI_Q: SRP_GEMM_LAUNCH(EPI_Q); break;
    default: SRP_GEMM_LAUNCH(EPI_ENC); break;
  }
#undef SRP_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace srp
