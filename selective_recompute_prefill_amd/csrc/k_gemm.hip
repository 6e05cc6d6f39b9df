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
// 2x2 blocks of 32x32x16 MFMA.
// ------------------------------------------------------------------------- //
constexpr int kBM16 = 128, kBK16 = 64, kLDA16 = kBK16 + 8;  // 144-byte LDS rows
constexpr int kStage16 = kBM16 * kLDA16;                    // elements per operand stage
constexpr int kLDC = kBN + 4;

template <int MODE>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __align__(16) uint16_t smem[4 * kStage16];  // A0 A1 B0 B1 (73,728 B)
  uint16_t *As = smem, *Bs = smem + 2 * kStage16;
  float *Cs = reinterpret_cast<float *>(smem);           // 128 x 132 fp32 (67,584 B)

  const int M = g.M_dev ? *g.M_dev : g.M_host;
  const int K = g.K, N = g.N;
  const int mt_n = (M + kBM16 - 1) / kBM16, nt_n = (N + kBN - 1) / kBN;
  const TileIter ti(mt_n * nt_n);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const uint16_t *A = (const uint16_t *)g.A, *B = (const uint16_t *)g.B;
  const int KT = K / kBK16;

  for (int lt = ti.loc;; lt += ti.per_x) {
    const int tile = ti.tile(lt);
    if (tile < 0) break;
    const int mt = tile / nt_n, nt = tile - mt * nt_n;
    const int m0 = mt * kBM16, n0 = nt * kBN;

    // per-thread global source rows for its 4 A and 4 B chunks (16 B each)
    const uint16_t *pa[4], *pb[4];
    int lds_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, r = c >> 3, kc = c & 7;
      const int m = m0 + r, n = n0 + r;
      pa[i] = nullptr;
      if (m < M) {
        const int row = g.a_rows ? g.a_rows[m] : m;
        pa[i] = A + (size_t)row * K + kc * 8;
      }
      pb[i] = n < N ? B + (size_t)n * K + kc * 8 : nullptr;
      lds_off[i] = r * kLDA16 + kc * 8;
    }
    uint4 ra[4], rb[4];
    auto gload = [&](int kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = pa[i] ? *reinterpret_cast<const uint4 *>(pa[i] + kt * kBK16) : make_uint4(0, 0, 0, 0);
        rb[i] = pb[i] ? *reinterpret_cast<const uint4 *>(pb[i] + kt * kBK16) : make_uint4(0, 0, 0, 0);
      }
    };
    auto sstore = [&](int st) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<uint4 *>(As + st * kStage16 + lds_off[i]) = ra[i];
        *reinterpret_cast<uint4 *>(Bs + st * kStage16 + lds_off[i]) = rb[i];
      }
    };

    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    gload(0);
    sstore(0);
    __syncthreads();
    const int fr = lane & 31, fk = (lane >> 5) * 8;
    for (int kt = 0; kt < KT; ++kt) {
      const int st = kt & 1;
      if (kt + 1 < KT) gload(kt + 1);
      const uint16_t *as = As + st * kStage16, *bs = Bs + st * kStage16;
#pragma unroll
      for (int ks = 0; ks < kBK16 / 16; ++ks) {
        bf16x8 af[2], bfr[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          af[i] = *reinterpret_cast<const bf16x8 *>(as + (wm * 64 + i * 32 + fr) * kLDA16 + ks * 16 + fk);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bfr[j] = *reinterpret_cast<const bf16x8 *>(bs + (wn * 64 + j * 32 + fr) * kLDA16 + ks * 16 + fk);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < KT) sstore(st ^ 1);
      __syncthreads();
    }
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
  // resident work-groups: 256 CUs x 2, rounded to a multiple of the 8 XCDs
  long grid = tiles < 512 ? tiles : 512;
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
