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

// Waves per work-group: one per (query head of the group, 32-row query
// sub-tile); groups with fewer than 4 heads take several sub-tiles so that at
// least 4 waves share each K/V tile.
__host__ __device__ constexpr int attn_subtiles(int G) { return G >= 4 ? 1 : (4 + G - 1) / G; }

#ifndef SRP_ATTN_KEYS
#define SRP_ATTN_KEYS 64
#endif
#ifndef SRP_ATTN_OCC
#define SRP_ATTN_OCC 2
#endif
constexpr int kBK = SRP_ATTN_KEYS;  // keys per LDS stage

template <int D, int W>
__global__ __launch_bounds__(64 * W, (W == 5 || W == 6) ? SRP_ATTN_OCC : 2) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KLD = D + 8;       // K tile row stride (elements)
  constexpr int VLD = kBK + 8;     // V^T tile row stride
  constexpr int KSZ = kBK * KLD, VSZ = D * VLD;
  constexpr int NT = 64 * W;
  constexpr int KCH = kBK * (D / 8);        // 16-byte chunks of a K tile
  constexpr int VCH = (kBK / 2) * (D / 8);  // (key pair, 8-wide d chunk) items of a V tile
  constexpr int KIT = (KCH + NT - 1) / NT, VIT = (VCH + NT - 1) / NT;
  __shared__ __align__(16) uint16_t lds[2 * (KSZ + VSZ)];

  const int n_tiles = *a.n_tiles;
  const int slot = blockIdx.x / a.nkv, g = blockIdx.x - slot * a.nkv;
  if (slot >= n_tiles) return;
  const int G = a.nh / a.nkv;
  const int q0 = a.tiles[3 * slot], nq = a.tiles[3 * slot + 1], r = a.tiles[3 * slot + 2];
  const int key_start = a.req_offsets[r];
  const int first_row = a.sel_idx[q0], last_row = a.sel_idx[q0 + nq - 1];
  const int key_end = last_row + 1;
  const int nblk = (key_end - key_start + kBK - 1) / kBK;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hw = w % G, qs = w / G;
  const int h = g * G + hw;
  const int qi = lane & 31, gph = lane >> 5;
  const int qidx = qs * 32 + qi;
  const bool qvalid = qidx < nq;
  const int qrow = qvalid ? a.sel_idx[q0 + qidx] : last_row;
  const size_t kvd = (size_t)a.nkv * D;
  const uint16_t *K = (const uint16_t *)a.k_cache + g * D;
  const uint16_t *V = (const uint16_t *)a.v_cache + g * D;

  // register-staged loads of the next K/V tile (K and V in separate phases so
  // only one of them is held in registers at a time)
  uint4 rk[KIT], rv0[VIT], rv1[VIT];
  auto kload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < KIT; ++i) {
      const int c = tid + NT * i;
      const int key = c / (D / 8), dc = c - key * (D / 8);
      const int krow = kb + key;
      rk[i] = (c < KCH && krow < key_end)
                  ? *reinterpret_cast<const uint4 *>(K + (size_t)krow * kvd + dc * 8)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto kstore = [&](int st) {
    uint16_t *Ks = lds + st * (KSZ + VSZ);
#pragma unroll
    for (int i = 0; i < KIT; ++i) {
      const int c = tid + NT * i;
      if (c < KCH) {
        const int key = c / (D / 8), dc = c - key * (D / 8);
        *reinterpret_cast<uint4 *>(Ks + key * KLD + dc * 8) = rk[i];
      }
    }
  };
  auto vload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int c = tid + NT * i;
      const int kp = c % (kBK / 2), dc = c / (kBK / 2);
      const int k0 = kb + 2 * kp;
      const bool ok = c < VCH;
      rv0[i] = (ok && k0 < key_end) ? *reinterpret_cast<const uint4 *>(V + (size_t)k0 * kvd + dc * 8)
                                    : make_uint4(0, 0, 0, 0);
      rv1[i] = (ok && k0 + 1 < key_end)
                   ? *reinterpret_cast<const uint4 *>(V + (size_t)(k0 + 1) * kvd + dc * 8)
                   : make_uint4(0, 0, 0, 0);
    }
  };
  // V transposed: 8 key pairs of one 8-wide d chunk as 32-bit words
  auto vstore = [&](int st) {
    uint16_t *Vt = lds + st * (KSZ + VSZ) + KSZ;
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int c = tid + NT * i;
      if (c < VCH) {
        const int kp = c % (kBK / 2), dc = c / (kBK / 2);
        const uint32_t x0[4] = {rv0[i].x, rv0[i].y, rv0[i].z, rv0[i].w};
        const uint32_t x1[4] = {rv1[i].x, rv1[i].y, rv1[i].z, rv1[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          *reinterpret_cast<uint32_t *>(Vt + (dc * 8 + 2 * j) * VLD + 2 * kp) =
              (x0[j] & 0xffffu) | (x1[j] << 16);
          *reinterpret_cast<uint32_t *>(Vt + (dc * 8 + 2 * j + 1) * VLD + 2 * kp) =
              (x0[j] >> 16) | (x1[j] & 0xffff0000u);
        }
      }
    }
  };

  bf16x8 qf[D / 16];
  {
    const uint16_t *qp = (const uint16_t *)a.q + ((size_t)(q0 + qidx) * a.nh + h) * D + gph * 8;
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
  // scores are already in base-2 units (queries carry log2(e)/sqrt(d)); m_ref is
  // the reference max of the exponentials, raised only when a block's max exceeds
  // it by more than 8, so probabilities stay below 2^8 and rescales are rare
  float m_ref = -INFINITY, l = 0.f;

  kload(key_start);
  vload(key_start);
  kstore(0);
  vstore(0);
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const int kb = key_start + blk * kBK;
    const int st = blk & 1;
    const bool more = blk + 1 < nblk;
    const uint16_t *Ks = lds + st * (KSZ + VSZ), *Vt = Ks + KSZ;
    const bool masked = kb + kBK - 1 > first_row;
    if (kBK == 32 && more) {
      kload(kb + kBK);
      vload(kb + kBK);
    }
#pragma unroll
    for (int kb2 = 0; kb2 < kBK / 32; ++kb2) {
      if (kBK == 64 && more) {
        if (kb2 == 0) kload(kb + kBK);
        else vload(kb + kBK);
      }
      // S^T[key][query] for 32 keys
      floatx16 s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Ks + (kb2 * 32 + qi) * KLD + ks * 16 + gph * 8);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
      }
      if (masked) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int krow = kb + kb2 * 32 + (e >> 2) * 8 + gph * 4 + (e & 3);
          if (krow > qrow) s[e] = -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const bool up = mx > m_ref + 8.f;
      if (__any(up)) {
        const float m_new = up ? mx : m_ref;
        const float alpha = exp2f(m_ref - m_new);
        m_ref = m_new;
        l *= alpha;
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[b][e] *= alpha;
      }
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(s[e] - m_ref);
        s[e] = p;
        rs += p;
      }
      l += rs + __shfl_xor(rs, 32, 64);

      // O^T += V^T P^T, 16 keys per step; P^T element j of lane l is key
      // 8*(j/4) + 4*(l/32) + j%4 of the step, matching the V^T fragment below
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x8 pf;
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[j] = (__bf16)s[hf * 8 + j];
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
      if (kBK == 64 && more) {
        if (kb2 == 0) kstore(st ^ 1);
        else vstore(st ^ 1);
      }
    }
    if (kBK == 32 && more) {
      kstore(st ^ 1);
      vstore(st ^ 1);
    }
    __syncthreads();
  }

  if (qvalid) {
    const float inv = 1.f / l;
    uint16_t *op = (uint16_t *)a.out + ((size_t)(q0 + qidx) * a.nh + h) * D;
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

int attn_tile_rows(int dtype, int nh, int nkv) {
  return dtype == SRP_BF16 ? 32 * attn_subtiles(nh / nkv) : 32;
}

template <int D>
static void launch_bf16(const AttnArgs &a, int W, dim3 grid, hipStream_t s) {
  switch (W) {
    case 4: hipLaunchKernelGGL((attn_bf16_kernel<D, 4>), grid, dim3(256), 0, s, a); break;
    case 5: hipLaunchKernelGGL((attn_bf16_kernel<D, 5>), grid, dim3(320), 0, s, a); break;
    case 6: hipLaunchKernelGGL((attn_bf16_kernel<D, 6>), grid, dim3(384), 0, s, a); break;
    case 7: hipLaunchKernelGGL((attn_bf16_kernel<D, 7>), grid, dim3(448), 0, s, a); break;
    default: hipLaunchKernelGGL((attn_bf16_kernel<D, 8>), grid, dim3(512), 0, s, a); break;
  }
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t s) {
  const int G = a.nh / a.nkv;
  const dim3 grid((unsigned)(a.max_tiles * a.nkv));
  if (a.dtype == SRP_BF16) {
    const int W = G * attn_subtiles(G);
    if (a.d == 128) launch_bf16<128>(a, W, grid, s);
    else launch_bf16<64>(a, W, grid, s);
  } else {
    const dim3 block((unsigned)(64 * G));
    if (a.d == 128) hipLaunchKernelGGL(attn_f32_kernel<128>, grid, block, 0, s, a);
    else hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace srp
