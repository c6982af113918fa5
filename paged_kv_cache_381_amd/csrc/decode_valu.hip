// PagedAttention decode, wavefront-reduction kernel (any KV type, G <= 16).
//
// Same computation as the matrix-core kernel [KV Cache 工程学 §15.5;
// 新一代 KV Cache 管理 §8.1]: scores of the new token's query against every
// cached key, fetched through the block table, a softmax over the whole
// context kept as a running maximum and sum, and the weighted sum of V.  It
// serves multi-head attention (one query head per kv head, where a group
// product is a matrix-vector product and gains nothing from matrix cores) and
// float32 caches.
//
// gfx950 mapping, per wave and 16-token block (one 16*D-element tile of K and
// one of V, each read as 16-byte units u = 64 i + lane, fully coalesced):
//   K tile [D/X][16][X]: lane holds token lane%16 for chunks 4i + lane/16, so
//     a score is an in-lane dot over X*D/(4X) elements plus a two-step
//     cross-row reduction (lanes l, l^16, l^32, l^48);
//   the block maximum is a DPP all-reduce inside a 16-lane row;
//   V tile [D][16]: lane holds X consecutive tokens of one d, so the weights
//     of those tokens are read back from a per-wave LDS line and the lane
//     accumulates out[d] directly; partial sums over token halves/quarters are
//     folded with one or two DPP steps at the end.
// The group's query rows are staged in LDS as float and shared by the W waves
// that split the partition's blocks; the waves merge through LDS.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace {

template <typename E>
__device__ __forceinline__ float unit_elem(const uint4 &u, int e);

template <>
__device__ __forceinline__ float unit_elem<uint16_t>(const uint4 &u, int e) {
  const uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}
template <>
__device__ __forceinline__ float unit_elem<float>(const uint4 &u, int e) {
  const uint32_t w = e == 0 ? u.x : e == 1 ? u.y : e == 2 ? u.z : u.w;
  return __uint_as_float(w);
}

template <typename E>
__device__ __forceinline__ float load_elem(const void *p, size_t i);
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const void *p, size_t i) {
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p)[i] << 16);
}
template <>
__device__ __forceinline__ float load_elem<float>(const void *p, size_t i) {
  return reinterpret_cast<const float *>(p)[i];
}

template <typename E, int D, int GP, int W>
__global__ __launch_bounds__(64 * W) void decode_valu_kernel(DecodeParams P) {
  constexpr int ES = sizeof(E);
  constexpr int X = 16 / ES;   // elements per 16-byte unit
  constexpr int NL = D * ES / 64;  // units per lane per tile (tile = D*ES units)
  constexpr bool QREG = GP * NL * X <= 64;
  extern __shared__ __align__(16) char smem[];
  float *q_lds = reinterpret_cast<float *>(smem);  // [GP][D]
  float *p_lds = q_lds + GP * D;                   // [W][GP][16]
  float *red_m = p_lds + W * GP * 16;              // [W][GP]
  float *red_l = red_m + W * GP;                   // [W][GP]
  float *red_o = red_l + W * GP;                   // [W][GP][D]

  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = P.G;
  const int n = clamp_len(P.ctx[b], P.max_blocks, P.max_ctx);
  const int t0 = part * P.part_tokens;
  float *out_bg = P.out + ((size_t)b * P.Hq + (size_t)g * G) * D;
  if (n == 0) {
    if (part == 0)
      for (int i = tid; i < G * D; i += 64 * W) out_bg[i] = 0.f;
    return;
  }
  if (t0 >= n) return;
  const int t1 = min(t0 + P.part_tokens, n);
  const int nparts_b = (n + P.part_tokens - 1) / P.part_tokens;

  const size_t qoff = ((size_t)b * P.Hq + (size_t)g * G) * D;
  for (int i = tid; i < GP * D; i += 64 * W) q_lds[i] = (i / D) < G ? load_elem<E>(P.q, qoff + i) : 0.f;
  __syncthreads();

  const int tok = lane & 15, row = lane >> 4;
  const int vpart = lane % ES;  // which X-token run of a V row this lane reads
  float qr[QREG ? GP : 1][QREG ? NL : 1][QREG ? X : 1];
  if constexpr (QREG) {
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int e = 0; e < X; ++e) qr[h][i][e] = q_lds[h * D + (4 * i + row) * X + e];
  }

  float m[GP], lsum[GP], acc[GP][NL];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i) acc[h][i] = 0.f;
  }

  const int32_t *tbl = P.tables + (size_t)b * P.max_blocks;
  const E *kpool = reinterpret_cast<const E *>(P.k_pool);
  const E *vpool = reinterpret_cast<const E *>(P.v_pool);
  float *pl = p_lds + w * GP * 16;
  const int jb1 = (t1 + 15) >> 4;

  for (int jb = (t0 >> 4) + w; jb < jb1; jb += W) {
    const int phys = clamp_block(tbl[jb], P.num_blocks);
    const size_t tile = ((size_t)phys * P.H + g) * 16 * D;
    const uint4 *kt = reinterpret_cast<const uint4 *>(kpool + tile);
    const uint4 *vt = reinterpret_cast<const uint4 *>(vpool + tile);
    uint4 ku[NL], vu[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) ku[i] = kt[64 * i + lane];
#pragma unroll
    for (int i = 0; i < NL; ++i) vu[i] = vt[64 * i + lane];

    const bool valid = jb * 16 + tok < n;
    float p[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int e = 0; e < X; ++e) {
          const float qv = QREG ? qr[QREG ? h : 0][QREG ? i : 0][QREG ? e : 0] : q_lds[h * D + (4 * i + row) * X + e];
          s += qv * unit_elem<E>(ku[i], e);
        }
      s = rows_sum4(s);
      s = valid ? s * P.scale_log2 : -INFINITY;
      const float mnew = fmaxf(m[h], row_max16(s));
      const float alpha = fast_exp2(m[h] - mnew);
      m[h] = mnew;
      p[h] = fast_exp2(s - mnew);
      lsum[h] = lsum[h] * alpha + p[h];
#pragma unroll
      for (int i = 0; i < NL; ++i) acc[h][i] *= alpha;
    }
    if (row == 0) {
#pragma unroll
      for (int h = 0; h < GP; ++h) pl[h * 16 + tok] = p[h];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int vtok0 = jb * 16 + vpart * X;
    const int nvalid = min(max(n - vtok0, 0), X);
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      float pw[X];
#pragma unroll
      for (int e = 0; e < X; ++e) pw[e] = pl[h * 16 + vpart * X + e];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        float a = acc[h][i];
#pragma unroll
        for (int e = 0; e < X; ++e) {
          const float v = unit_elem<E>(vu[i], e);
          a += (e < nvalid) ? pw[e] * v : 0.f;  // select: a NaN past the end must not leak
        }
        acc[h][i] = a;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

  // Fold token partial sums: lanes sharing a d differ in their low log2(ES) bits.
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    lsum[h] = row_sum16(lsum[h]);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      acc[h][i] += dpp<PKV_DPP_XOR1>(acc[h][i]);
      if constexpr (ES == 4) acc[h][i] += dpp<PKV_DPP_XOR2>(acc[h][i]);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      red_m[w * GP + h] = m[h];
      red_l[w * GP + h] = lsum[h];
    }
  }
  if (vpart == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
      for (int i = 0; i < NL; ++i) red_o[((size_t)w * GP + h) * D + (64 * i + lane) / ES] = acc[h][i];
  }
  __syncthreads();

  for (int i = tid; i < G * D; i += 64 * W) {
    const int h = i / D, d = i - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < W; ++v) M = fmaxf(M, red_m[v * GP + h]);
    float a = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const float f = fast_exp2(red_m[v * GP + h] - M);
      a += f * red_o[((size_t)v * GP + h) * D + d];
      L += f * red_l[v * GP + h];
    }
    if (nparts_b == 1) {
      out_bg[(size_t)h * D + d] = a / L;
    } else {
      const size_t r = ((size_t)b * P.Hq + (size_t)g * G + h) * P.num_parts + part;
      P.ws_o[r * D + d] = a;
      if (d == 0) {
        P.ws_ml[2 * r] = M;
        P.ws_ml[2 * r + 1] = L;
      }
    }
  }
}

constexpr int kWaves = 4;

template <typename E, int D, int GP>
int launch(const pkv_decode_args &a, const DecodeParams &p) {
  const size_t lds = (size_t)(GP * D + kWaves * GP * 16 + 2 * kWaves * GP + kWaves * GP * D) * sizeof(float);
  dim3 grid(a.num_parts, a.L->num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_valu_kernel<E, D, GP, kWaves>), grid, dim3(64 * kWaves), lds,
                     reinterpret_cast<hipStream_t>(a.stream), p);
  return (int)hipGetLastError();
}

template <typename E, int D>
int launch_g(const pkv_decode_args &a, const DecodeParams &p) {
  if (p.G <= 1) return launch<E, D, 1>(a, p);
  if (p.G <= 2) return launch<E, D, 2>(a, p);
  if (p.G <= 4) return launch<E, D, 4>(a, p);
  if (p.G <= 8) return launch<E, D, 8>(a, p);
  return launch<E, D, 16>(a, p);
}

}  // namespace

int pkv_launch_decode_valu(const pkv_decode_args &a) {
  DecodeParams p{a.out, a.q, a.k_pool, a.v_pool, a.tables, a.ctx, a.ws_o, a.ws_ml,
                 a.L->num_blocks, a.L->num_kv_heads, a.num_q_heads, a.num_q_heads / a.L->num_kv_heads,
                 a.max_blocks, a.max_ctx, a.part_tokens, a.num_parts, a.scale_log2};
  const bool bf = a.L->kv_dtype == PKV_BF16;
  if (a.L->head_dim == 128) return bf ? launch_g<uint16_t, 128>(a, p) : launch_g<float, 128>(a, p);
  return bf ? launch_g<uint16_t, 64>(a, p) : launch_g<float, 64>(a, p);
}
