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
#include <type_traits>

#include "kernels.hpp"

namespace srp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// Calls f(integral_constant<int, i>) for i = 0..N-1, so array indices inside f
// are compile-time constants (register arrays stay in registers).
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// Waves per work-group: one per (query head of the group, 32-row query
// sub-tile); groups of fewer than 5 heads take several sub-tiles so that 6-8
// waves (2 per SIMD) share each K/V tile.
__host__ __device__ constexpr int attn_subtiles(int G) { return G >= 5 ? 1 : (G == 3 ? 2 : 8 / G); }

constexpr int kBK = 64;  // keys per LDS stage

template <int D, int W>
__global__ __launch_bounds__(64 * W, 2) void attn_bf16_kernel(AttnArgs a) {
  constexpr int KLD = D + 8;    // K tile row stride (elements, 16-byte padded rows)
  constexpr int VLD = kBK + 8;  // V^T tile row stride
  constexpr int KSZ = kBK * KLD, VSZ = D * VLD;
  constexpr int NT = 64 * W;
  constexpr int KCH = kBK * (D / 8);        // 16-byte chunks of a K tile
  constexpr int VCH = (kBK / 2) * (D / 8);  // (key pair, 8-wide d chunk) items of a V tile
  constexpr int KIT = (KCH + NT - 1) / NT, VIT = (VCH + NT - 1) / NT;
  __shared__ __align__(16) uint16_t lds[2 * (KSZ + VSZ)];
  __shared__ uint4 qlds[W * (D / 16) * 64];  // each lane's Q fragments, in fragment order

  const int n_tiles = *a.n_tiles;
  const int slot = blockIdx.x / a.nkv, g = blockIdx.x - slot * a.nkv;
  if (slot >= n_tiles) return;
  const int G = a.nh / a.nkv;
  const int q0 = a.tiles[3 * slot], nq = a.tiles[3 * slot + 1], r = a.tiles[3 * slot + 2];
  const int key_start = a.req_offsets[r];
  const int first_row = a.sel_idx[q0], last_row = a.sel_idx[q0 + nq - 1];
  const int key_end = last_row + 1;
  const int nblk = (key_end - key_start + kBK - 1) / kBK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int hw = w % G, qs = w / G;
  const int h = g * G + hw;
  const int qi = lane & 31, gph = lane >> 5;
  const int qidx = qs * 32 + qi;
  const bool qvalid = qidx < nq;
  const int qrow = qvalid ? a.sel_idx[q0 + qidx] : last_row;
  const int kvd = a.nkv * D;
  const size_t row_bytes = (size_t)kvd * 2;
  const char *Kg = (const char *)a.k_cache + (size_t)g * D * 2;
  const char *Vg = (const char *)a.v_cache + (size_t)g * D * 2;

  // Loader: thread chunk i covers K chunk c = tid + NT*i, i.e. key tid/(D/8) +
  // i*NT/(D/8) at d chunk tid%(D/8), and V item c, i.e. key pair tid%32 at d chunk
  // tid/32 + i*NT/32. NT is a multiple of both widths, so each offset is one
  // per-thread constant plus a uniform step, and whether chunk i exists is uniform
  // per wave (KCH, VCH and NT are multiples of 64).
  constexpr int KSTEP = NT / (D / 8);  // keys per K chunk step
  constexpr int VSTEP = NT / (kBK / 2);  // d chunks per V item step
  const int kkey0 = tid / (D / 8), kdc = tid % (D / 8);
  const int vkp = tid % (kBK / 2), vdc0 = tid / (kBK / 2);
  const uint32_t koff0 = (uint32_t)(kkey0 * row_bytes + kdc * 16);
  const uint32_t voff0 = (uint32_t)(2 * vkp * row_bytes + vdc0 * 16);
  u32x4 rk[KIT], rv0[VIT], rv1[VIT];
  auto load_next = [&](int kb) __attribute__((always_inline)) {
    const char *kbase = Kg + (size_t)kb * row_bytes, *vbase = Vg + (size_t)kb * row_bytes;
    if (kb + kBK <= key_end) {
      static_for<KIT>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        if (w * 64 + NT * i < KCH)
          rk[i] = *reinterpret_cast<const u32x4 *>(kbase + (size_t)i * KSTEP * row_bytes + koff0);
      });
      static_for<VIT>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        if (w * 64 + NT * i < VCH) {
          const char *p = vbase + (size_t)i * VSTEP * 16 + voff0;
          rv0[i] = *reinterpret_cast<const u32x4 *>(p);
          rv1[i] = *reinterpret_cast<const u32x4 *>(p + row_bytes);
        }
      });
    } else {
      // last, partial tile: rows past key_end are clamped to the last valid row;
      // every such key lies after every query of the tile and is masked
      const int lastk = key_end - 1 - kb;
      static_for<KIT>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        if (w * 64 + NT * i < KCH) {
          const int key = min(kkey0 + i * KSTEP, lastk);
          rk[i] = *reinterpret_cast<const u32x4 *>(kbase + (size_t)key * row_bytes + kdc * 16);
        }
      });
      static_for<VIT>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        if (w * 64 + NT * i < VCH) {
          const char *p = vbase + (size_t)(vdc0 + i * VSTEP) * 16;
          rv0[i] = *reinterpret_cast<const u32x4 *>(p + (size_t)min(2 * vkp, lastk) * row_bytes);
          rv1[i] = *reinterpret_cast<const u32x4 *>(p + (size_t)min(2 * vkp + 1, lastk) * row_bytes);
        }
      });
    }
  };
  auto store_next = [&](int st) __attribute__((always_inline)) {
    uint16_t *Ks = lds + st * (KSZ + VSZ), *Vt = Ks + KSZ;
    static_for<KIT>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if (w * 64 + NT * i < KCH)
        *reinterpret_cast<u32x4 *>(Ks + (kkey0 + i * KSTEP) * KLD + kdc * 8) = rk[i];
    });
    // V transposed: word j of two keys -> d rows 2j (low halves), 2j+1 (high halves)
    static_for<VIT>([&](auto I) __attribute__((always_inline)) {
      constexpr int i = decltype(I)::value;
      if (w * 64 + NT * i < VCH) {
        uint16_t *vt = Vt + (vdc0 + i * VSTEP) * 8 * VLD + 2 * vkp;
        const u32x4 a0 = rv0[i], a1 = rv1[i];
        *reinterpret_cast<uint32_t *>(vt + 0 * VLD) = __builtin_amdgcn_perm(a1.x, a0.x, 0x05040100u);
        *reinterpret_cast<uint32_t *>(vt + 1 * VLD) = __builtin_amdgcn_perm(a1.x, a0.x, 0x07060302u);
        *reinterpret_cast<uint32_t *>(vt + 2 * VLD) = __builtin_amdgcn_perm(a1.y, a0.y, 0x05040100u);
        *reinterpret_cast<uint32_t *>(vt + 3 * VLD) = __builtin_amdgcn_perm(a1.y, a0.y, 0x07060302u);
        *reinterpret_cast<uint32_t *>(vt + 4 * VLD) = __builtin_amdgcn_perm(a1.z, a0.z, 0x05040100u);
        *reinterpret_cast<uint32_t *>(vt + 5 * VLD) = __builtin_amdgcn_perm(a1.z, a0.z, 0x07060302u);
        *reinterpret_cast<uint32_t *>(vt + 6 * VLD) = __builtin_amdgcn_perm(a1.w, a0.w, 0x05040100u);
        *reinterpret_cast<uint32_t *>(vt + 7 * VLD) = __builtin_amdgcn_perm(a1.w, a0.w, 0x07060302u);
      }
    });
  };

  // Q fragments (B operand of S^T = K Q^T): lane holds query qi, d range
  // ks*16 + gph*8 .. +8; parked in LDS to keep registers for the accumulators
  uint4 *qmine = qlds + w * (D / 16) * 64 + lane;
  {
    const uint16_t *qp = (const uint16_t *)a.q + ((size_t)(q0 + qidx) * a.nh + h) * D + gph * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      qmine[ks * 64] = qvalid ? *reinterpret_cast<const uint4 *>(qp + ks * 16) : make_uint4(0, 0, 0, 0);
  }
  floatx16 acc[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
  // Scores are in base-2 units (queries carry log2(e)/sqrt(d)). The score
  // accumulators start at -m, so they come out of the MFMA already relative to
  // the reference max m, which is raised only when a half-block's max exceeds
  // it by more than 8: probabilities stay below 2^8 and rescales are rare.
  float m = 0.f, l = 0.f;
  bool first = true;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  load_next(key_start);
  store_next(0);
  __syncthreads();
  for (int blk = 0; blk < nblk; ++blk) {
    const int kb = key_start + blk * kBK;
    const int st = blk & 1;
    const bool more = blk + 1 < nblk;
    const uint16_t *Ks = lds + st * (KSZ + VSZ), *Vt = Ks + KSZ;
    if (more) load_next(kb + kBK);

    // S^T[key][query] - m for both 32-key halves, two independent MFMA chains
    floatx16 s[2];
    const float c0 = first ? 0.f : -m;
#pragma unroll
    for (int e = 0; e < 16; ++e) { s[0][e] = c0; s[1][e] = c0; }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      uint4 qt = qmine[ks * 64];
      const bf16x8 qf = *reinterpret_cast<bf16x8 *>(&qt);
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(Ks + (hb * 32 + qi) * KLD + ks * 16 + gph * 8);
        s[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf, s[hb], 0, 0, 0);
      }
    }
    const bool masked = kb + kBK - 1 > first_row;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      if (masked) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int krow = kb + hb * 32 + (e >> 2) * 8 + gph * 4 + (e & 3);
          if (krow > qrow) s[hb][e] = -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[hb][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (first) {
        // the first half-block sets the reference max (its first key is
        // visible to every query, so mx is finite)
        first = false;
        m = mx;
#pragma unroll
        for (int e = 0; e < 16; ++e) { s[0][e] -= mx; s[1][e] -= mx; }
      } else {
        const bool up = mx > 8.f;
        if (__any(up)) {
          const float dlt = up ? mx : 0.f;
          const float alpha = __builtin_amdgcn_exp2f(-dlt);
          m += dlt;
          l *= alpha;
#pragma unroll
          for (int b = 0; b < D / 32; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[b][e] *= alpha;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            s[hb][e] -= dlt;
            if (hb == 0) s[1][e] -= dlt;
          }
        }
      }
      // probabilities in bf16 (the PV operand); the row sum uses the same
      // rounded values
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        bf16x8 pf;
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[j] = (__bf16)__builtin_amdgcn_exp2f(s[hb][hf * 8 + j]);
        float rs = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x2 pr = {pf[2 * j], pf[2 * j + 1]};
          rs = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, rs, false);
        }
        l += rs + __shfl_xor(rs, 32, 64);
        // O^T += V^T P^T over 16 keys; P^T element j of lane l is key
        // 8*(j/4) + 4*(l/32) + j%4 of the step, matching the V^T fragment
        const int kbase = hb * 32 + hf * 16 + gph * 4;
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
    if (more) store_next(st ^ 1);
    __syncthreads();
  }

  if (qvalid) {
    const float inv = 1.f / l;
    uint16_t *op = (uint16_t *)a.out + ((size_t)(q0 + qidx) * a.nh + h) * D;
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
