// Gathered-query causal GQA flash attention over the fused cache (gfx950).
//
// Work-group = (tile of up to 32 selected rows of one request, KV head g); one
// wave per query head of the group, so each K/V tile staged in LDS serves all
// nh/nkv heads that read it. The bf16 kernel computes S^T = K Q^T and
// O^T = V^T P^T with v_mfma_f32_32x32x16_bf16: in that orientation a lane holds
// one query's column, so the online-softmax max/sum need only one cross-lane step
// (lanes l and l^32) and the rescale of O is per lane. The probabilities are
// reused in registers as the B operand of the PV product, so V is staged in LDS
// transposed. Causality is by row: positions rise strictly inside a request.
#include "kernels.hpp"

namespace srp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
__global__ __launch_bounds__(512) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KLD = D + 8;   // K tile row stride (elements)
  constexpr int VLD = 64 + 8;  // V^T tile row stride
  __shared__ __align__(16) uint16_t Ks[64 * KLD];
  __shared__ __align__(16) uint16_t Vt[D * VLD];

  const int n_tiles = *a.n_tiles;
  const int slot = blockIdx.x / a.nkv, g = blockIdx.x - slot * a.nkv;
  if (slot >= n_tiles) return;
  const int G = a.nh / a.nkv;
  const int q0 = a.tiles[3 * slot], nq = a.tiles[3 * slot + 1], r = a.tiles[3 * slot + 2];
  const int key_start = a.req_offsets[r];
  const int first_row = a.sel_idx[q0], last_row = a.sel_idx[q0 + nq - 1];
  const int key_end = last_row + 1;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nthr = blockDim.x;
  const int h = g * G + w;
  const int qi = lane & 31, gph = lane >> 5;
  const bool qvalid = qi < nq;
  const int qrow = qvalid ? a.sel_idx[q0 + qi] : last_row;
  const size_t kvd = (size_t)a.nkv * D;
  const uint16_t *K = (const uint16_t *)a.k_cache + g * D;
  const uint16_t *V = (const uint16_t *)a.v_cache + g * D;

  bf16x8 qf[D / 16];
  {
    const uint16_t *qp = (const uint16_t *)a.q + ((size_t)(q0 + qi) * a.nh + h) * D + gph * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      uint4 t = qvalid ? *reinterpret_cast<const uint4 *>(qp + ks * 16) : make_uint4(0, 0, 0, 0);
      qf[ks] = *reinterpret_cast<bf16x8 *>(&t);
    }
  }
  floatx16 acc[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float scale = kLog2e / sqrtf((float)D);

  for (int kb = key_start; kb < key_end; kb += 64) {
    __syncthreads();
    // K tile: 64 keys x D, 16-byte chunks, chunk index fastest along d
    for (int c = tid; c < 64 * (D / 8); c += nthr) {
      const int key = c / (D / 8), dc = c - key * (D / 8);
      const int krow = kb + key;
      uint4 v = krow < key_end ? *reinterpret_cast<const uint4 *>(K + (size_t)krow * kvd + dc * 8)
                               : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4 *>(Ks + key * KLD + dc * 8) = v;
    }
    // V tile, transposed: a thread takes two keys of one 8-wide d chunk and
    // writes 8 key pairs as 32-bit words
    for (int c = tid; c < 32 * (D / 8); c += nthr) {
      const int kp = c & 31, dc = c >> 5;
      const int k0 = kb + 2 * kp;
      uint4 v0 = k0 < key_end ? *reinterpret_cast<const uint4 *>(V + (size_t)k0 * kvd + dc * 8)
                              : make_uint4(0, 0, 0, 0);
      uint4 v1 = k0 + 1 < key_end ? *reinterpret_cast<const uint4 *>(V + (size_t)(k0 + 1) * kvd + dc * 8)
                                  : make_uint4(0, 0, 0, 0);
      const uint32_t x0[4] = {v0.x, v0.y, v0.z, v0.w};
      const uint32_t x1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = (x0[i] & 0xffffu) | (x1[i] << 16);
        const uint32_t hi = (x0[i] >> 16) | (x1[i] & 0xffff0000u);
        *reinterpret_cast<uint32_t *>(Vt + (dc * 8 + 2 * i) * VLD + 2 * kp) = lo;
        *reinterpret_cast<uint32_t *>(Vt + (dc * 8 + 2 * i + 1) * VLD + 2 * kp) = hi;
      }
    }
    __syncthreads();

    // S^T[key][query] for two 32-key halves
    floatx16 s[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb2][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Ks + (kb2 * 32 + qi) * KLD + ks * 16 + gph * 8);
        s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kb2], 0, 0, 0);
      }
    }
    const bool need_mask = kb + 63 > first_row;
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float v = s[kb2][e] * scale;
        if (need_mask) {
          const int krow = kb + kb2 * 32 + (e >> 2) * 8 + gph * 4 + (e & 3);
          if (krow > qrow) v = -INFINITY;
        }
        s[kb2][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m, mx);
    const float alpha = exp2f(m - m_new);
    float rs = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(s[kb2][e] - m_new);
        s[kb2][e] = p;
        rs += p;
      }
    rs += __shfl_xor(rs, 32, 64);
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[b][e] *= alpha;

    // O^T += V^T P^T, 16 keys per step; P^T element j of lane l is key
    // 8*(j/4) + 4*(l/32) + j%4 of the step, matching the V^T fragment below
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kb2 = t >> 1, hf = t & 1;
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = (__bf16)s[kb2][hf * 8 + j];
      const int kbase = kb2 * 32 + hf * 16 + gph * 4;
#pragma unroll
      for (int b = 0; b < D / 32; ++b) {
        const uint16_t *vr = Vt + (b * 32 + qi) * VLD + kbase;
        uint2 lo = *reinterpret_cast<const uint2 *>(vr);
        uint2 hi = *reinterpret_cast<const uint2 *>(vr + 8);
        uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
        const bf16x8 vf = *reinterpret_cast<bf16x8 *>(&vv);
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[b], 0, 0, 0);
      }
    }
  }

  if (qvalid) {
    const float inv = 1.f / l;
    uint16_t *op = (uint16_t *)a.out + ((size_t)(q0 + qi) * a.nh + h) * D;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = acc[b][e4 * 4 + i] * inv;
        st4(op + b * 32 + e4 * 8 + gph * 4, v);
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

hipError_t launch_attention(const AttnArgs &a, hipStream_t s) {
  const int G = a.nh / a.nkv;
  const dim3 grid((unsigned)(a.max_tiles * a.nkv)), block((unsigned)(64 * G));
  if (a.dtype == SRP_BF16) {
    if (a.d == 128) hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, block, 0, s, a);
  } else {
    if (a.d == 128) hipLaunchKernelGGL(attn_f32_kernel<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace srp
