// Streaming kernels outside the projection: standalone positional recovery of the
// cached keys, and the residual + RMSNorm step between stacked layers (gfx950).
#include "kernels.hpp"

namespace srp {

// K[j] <- R(pos_j - src_j) K[j] for cached rows. One thread per 16-byte piece of
// the first half of a head and the matching piece of the second half (8 rotation
// pairs in bf16, 4 in fp32): consecutive threads cover consecutive pieces, so a
// row streams coalesced. The rotation index comes from row_delta when the caller
// has it (kFresh: no cache), else from the chunk layout.
__device__ __forceinline__ void ld16(const uint16_t *p, float v[8]) {
  const uint4 t = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = __uint_as_float(w[k] << 16);
    v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void st16(uint16_t *p, const float v[8]) {
  uint4 t;
  t.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  t.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  t.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
  t.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
  *reinterpret_cast<uint4 *>(p) = t;
}
__device__ __forceinline__ void ld16(const float *p, float v[4]) { ld4(p, v); }
__device__ __forceinline__ void st16(float *p, const float v[4]) { st4(p, v); }

template <typename T>
__global__ __launch_bounds__(256) void rerotate_kernel(int T_rows, int nkv, int d,
                                                      const int32_t *row_delta, const int32_t *row_slot,
                                                      PagedMap pm, const int32_t *chunk_offsets, int n_chunks,
                                                      const int32_t *chunk_src_pos,
                                                      const int32_t *positions, const uint8_t *skip,
                                                      RopeTable rt, T *k_cache) {
  constexpr int P = 16 / sizeof(T);  // rotation pairs per thread
  const int half = d >> 1, per_head = half / P, per_row = nkv * per_head;
  const int n = T_rows * per_row;
  for (int it = blockIdx.x * blockDim.x + threadIdx.x; it < n; it += gridDim.x * blockDim.x) {
    const int j = it / per_row;
    const int rem = it - j * per_row;
    const int gh = rem / per_head, i0 = (rem - gh * per_head) * P;
    int delta, cr = j;  // rotation index, cache row
    if (row_delta) {
      delta = row_delta[j];
      if (delta == kFresh) continue;
      if (row_slot) cr = row_slot[j];
    } else {
      const int c = upper_index(chunk_offsets, n_chunks + 1, j);
      const int src0 = chunk_src_pos[c];
      if (src0 < 0) continue;
      delta = positions[j] - (src0 + j - chunk_offsets[c]);
      if (pm.block_rows > 0) cr = paged_row(pm, c, j - chunk_offsets[c]);
    }
    if (delta == 0 || (skip && skip[j])) continue;
    T *p = k_cache + ((size_t)cr * nkv + gh) * d;
    float a[P], b[P];
    ld16(p + i0, a);
    ld16(p + half + i0, b);
#pragma unroll
    for (int q = 0; q < P; q += 4) rope4(a + q, b + q, rt, delta, i0 + q);
    st16(p + i0, a);
    st16(p + half + i0, b);
  }
}

hipError_t launch_rerotate(int dtype, int T, int nkv, int d, const int32_t *row_delta,
                           const int32_t *row_slot, const PagedMap &pm, const int32_t *chunk_offsets,
                           int n_chunks, const int32_t *chunk_src_pos, const int32_t *positions,
                           const uint8_t *skip, const RopeTable &rt, void *k_cache, hipStream_t s) {
  const int P = dtype == SRP_BF16 ? 8 : 4;
  const long n = (long)T * nkv * (d / 2 / P);
  if (n <= 0) return hipSuccess;
  if (n > INT_MAX) return hipErrorInvalidValue;  // the kernel indexes pieces with int
  long grid = (n + 255) / 256;
  grid = grid < 8192 ? grid : 8192;
  if (dtype == SRP_BF16)
    hipLaunchKernelGGL(rerotate_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, s, T, nkv, d,
                       row_delta, row_slot, pm, chunk_offsets, n_chunks, chunk_src_pos, positions, skip,
                       rt, (uint16_t *)k_cache);
  else
    hipLaunchKernelGGL(rerotate_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s, T, nkv, d,
                       row_delta, row_slot, pm, chunk_offsets, n_chunks, chunk_src_pos, positions, skip,
                       rt, (float *)k_cache);
  return hipGetLastError();
}

// dst[j] = src[row_slot[j]], rows of row_bytes (a multiple of 16): one wave per
// row, 16 bytes per lane and step.
__global__ __launch_bounds__(256) void gather_rows_kernel(int T_rows, int row_chunks, const int32_t *row_slot,
                                                         const uint4 *src, uint4 *dst) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  for (int j = wave; j < T_rows; j += nwaves) {
    const size_t from = (size_t)row_slot[j] * row_chunks, to = (size_t)j * row_chunks;
    for (int c = lane; c < row_chunks; c += 64) dst[to + c] = src[from + c];
  }
}

hipError_t launch_gather_rows(int T, size_t row_bytes, const int32_t *row_slot, const void *src,
                              void *dst, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  int grid = (T * 64 + 255) / 256;
  grid = grid < 4096 ? grid : 4096;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(grid), dim3(256), 0, s, T, (int)(row_bytes / 16), row_slot,
                     (const uint4 *)src, (uint4 *)dst);
  return hipGetLastError();
}

// hidden[j] <- y / sqrt(mean(y^2) + eps), y = hidden[j] + attn[s], j = sel_idx[s].
// One work-group per selected row; fixed-order reduction. A thread takes 8
// consecutive elements per 2048 (16-byte loads); rows of up to kNormRegs * 2048
// elements keep y in registers between the sum and the scaling, longer ones load
// it again.
constexpr int kNormRegs = 4;
__device__ __forceinline__ void ld8(const uint16_t *p, float v[8]) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = __uint_as_float(w[k] << 16);
    v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void ld8(const float *p, float v[8]) {
  const float4 a = *reinterpret_cast<const float4 *>(p), b = *reinterpret_cast<const float4 *>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void st8(uint16_t *p, const float v[8]) {
  st4(p, v);
  st4(p + 4, v + 4);
}
__device__ __forceinline__ void st8(float *p, const float v[8]) {
  st4(p, v);
  st4(p + 4, v + 4);
}

template <typename T>
__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(int H, T *hidden, const T *attn,
                                                              const int32_t *sel_idx,
                                                              const int32_t *total_dev, float eps) {
  __shared__ float red[4];
  const int total = *total_dev;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool in_regs = H <= kNormRegs * 2048;
  for (int s = blockIdx.x; s < total; s += gridDim.x) {
    const int j = sel_idx[s];
    T *x = hidden + (size_t)j * H;
    const T *o = attn + (size_t)s * H;
    float ss = 0.f;
    float y[kNormRegs][8];
    if (in_regs) {
      // every load issued before the first use (past the row end: a valid element,
      // its value dropped below)
      float a[kNormRegs][8], b[kNormRegs][8];
#pragma unroll
      for (int c = 0; c < kNormRegs; ++c) {
        const int i = min(tid * 8 + c * 2048, H - 8);
        ld8(x + i, a[c]);
        ld8(o + i, b[c]);
      }
#pragma unroll
      for (int c = 0; c < kNormRegs; ++c) {
        const int i = tid * 8 + c * 2048;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          y[c][k] = i < H ? a[c][k] + b[c][k] : 0.f;
          ss = fmaf(y[c][k], y[c][k], ss);
        }
      }
    } else {
      for (int i = tid * 8; i < H; i += 2048) {
        float a[8], b[8];
        ld8(x + i, a);
        ld8(o + i, b);
#pragma unroll
        for (int k = 0; k < 8; ++k) { const float v = a[k] + b[k]; ss = fmaf(v, v, ss); }
      }
    }
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if (lane == 0) red[w] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float sc = 1.f / sqrtf(tot / (float)H + eps);
    if (in_regs) {
#pragma unroll
      for (int c = 0; c < kNormRegs; ++c) {
        const int i = tid * 8 + c * 2048;
        if (i < H) {
#pragma unroll
          for (int k = 0; k < 8; ++k) y[c][k] *= sc;
          st8(x + i, y[c]);
        }
      }
    } else {
      for (int i = tid * 8; i < H; i += 2048) {
        float a[8], b[8];
        ld8(x + i, a);
        ld8(o + i, b);
#pragma unroll
        for (int k = 0; k < 8; ++k) a[k] = (a[k] + b[k]) * sc;
        st8(x + i, a);
      }
    }
    __syncthreads();
  }
}

hipError_t launch_residual_rmsnorm(int dtype, int H, void *hidden, const void *attn,
                                   const int32_t *sel_idx, const int32_t *total_dev, int cap,
                                   float eps, hipStream_t s) {
  if (cap <= 0) return hipSuccess;
  const int grid = cap < 2048 ? cap : 2048;
  if (dtype == SRP_BF16)
    hipLaunchKernelGGL(residual_rmsnorm_kernel<uint16_t>, dim3(grid), dim3(256), 0, s, H,
                       (uint16_t *)hidden, (const uint16_t *)attn, sel_idx, total_dev, eps);
  else
    hipLaunchKernelGGL(residual_rmsnorm_kernel<float>, dim3(grid), dim3(256), 0, s, H,
                       (float *)hidden, (const float *)attn, sel_idx, total_dev, eps);
  return hipGetLastError();
}

}  // namespace srp
