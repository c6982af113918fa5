// Split-context merge of the decode kernels' partial results.
//
// A context cut between waves of the balanced split (pkv_device.h) leaves one
// partial per wave: its running maximum m_i (base 2), weight sum l_i and
// unnormalised output o_i.  The whole-context softmax is recovered with
// M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i - M) / L, which is
// exact algebra (log-sum-exp), so the result equals a single softmax over all
// tokens.
//
// The partials of segment (g, b) are those of the waves whose shares overlap
// the segment's chunks, stored in share order.  The schedule header written by
// the decode kernel gives the chunk scan, the number of waves used and the
// region bounds, from which the segment's position and its first and last
// wave follow exactly as in the decode kernel.  Segments held by one wave, and empty sequences, were
// written by the decode kernel and are skipped here.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace {

// Sum over the 64 lanes in registers: DPP within each 16-lane row, then the
// gfx950 lane swaps across rows (no LDS round trip).
__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum16(x);
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D>
__global__ __launch_bounds__(64) void merge_kernel(SplitParams P) {
  const int bh = blockIdx.x;
  const int b = bh / P.Hq, h = bh - b * P.Hq, g = h / P.G;
  const int64_t c_tot = (int64_t)P.H * P.ws_hdr[0];
  const int nwe = P.ws_hdr[1];
  const int32_t *s_incl = P.ws_hdr + PKV_HDR_INTS;
  const int cnt = s_incl[b] - (b ? s_incl[b - 1] : 0);
  if (cnt == 0 || c_tot == 0) return;
  const int64_t seg0 = (int64_t)g * P.ws_hdr[0] + (s_incl[b] - cnt);
  Regions rg;
  rg.C = c_tot;
  rg.nwe = nwe;
  rg.nr = P.ws_hdr[2];
  rg.wpr = nwe / rg.nr;
  rg.bounds = reinterpret_cast<const int64_t *>(P.ws_hdr + 4);
  const int w0 = rg.wave_of(seg0), w1 = rg.wave_of(seg0 + cnt - 1);
  const int np = min(w1 - w0 + 1, P.maxp);
  if (np <= 1) return;
  const size_t row = (size_t)bh * P.maxp;
  const float2 *ml = reinterpret_cast<const float2 *>(P.ws_ml) + row;
  const float *o = P.ws_o + row * D;
  const int lane = threadIdx.x;
  // The partials' maxima and weighted sums, 64 partials at a time across the
  // lanes (one round trip per 64, not one per partial).
  float M = -INFINITY;
  for (int i = lane; i < np; i += 64) M = fmaxf(M, ml[i].x);
  M = rows_max4_swap(row_max16(M));
  float L = 0.f;
  float acc[D / 64];
#pragma unroll
  for (int k = 0; k < D / 64; ++k) acc[k] = 0.f;
  for (int i0 = 0; i0 < np; i0 += 64) {
    const int n = min(np - i0, 64);
    float f = 0.f;  // lane j: weight of partial i0 + j
    if (lane < n) {
      const float2 mi = ml[i0 + lane];
      f = fast_exp2(mi.x - M);
      L += mi.y * f;
    }
    // Output rows four partials at a time, so their loads are in flight
    // together; the sum runs over the partials in order.
    int j = 0;
    for (; j + 4 <= n; j += 4) {
      float v[4][D / 64];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < D / 64; ++k) v[u][k] = o[(size_t)(i0 + j + u) * D + 64 * k + lane];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float fu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j + u));
#pragma unroll
        for (int k = 0; k < D / 64; ++k) acc[k] += v[u][k] * fu;
      }
    }
    for (; j < n; ++j) {
      const float fj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j));
#pragma unroll
      for (int k = 0; k < D / 64; ++k) acc[k] += o[(size_t)(i0 + j) * D + 64 * k + lane] * fj;
    }
  }
  L = wave_sum(L);
  const float inv = 1.f / L;
#pragma unroll
  for (int k = 0; k < D / 64; ++k) P.out[(size_t)bh * D + 64 * k + lane] = acc[k] * inv;
}

}  // namespace

int pkv_launch_merge(const pkv_decode_args &a) {
  const SplitParams p = pkv_split_params(a);
  dim3 grid(a.num_seqs * a.num_q_heads);
  if (a.L->head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(64), 0, reinterpret_cast<hipStream_t>(a.stream), p);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(64), 0, reinterpret_cast<hipStream_t>(a.stream), p);
  return (int)hipGetLastError();
}
