// Split-context merge of the decode kernels' partial results.
//
// A context cut between waves of the balanced split (pkv_device.h) leaves one
// partial per wave: its running maximum m_i (base 2), weight sum l_i and
// unnormalised output o_i.  The whole-context softmax is recovered with
// M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i - M) / L, which is
// exact algebra (log-sum-exp), so the result equals a single softmax over all
// tokens.
//
// One wave per (sequence, kv head) segment.  The schedule header written by
// the decode kernel gives the chunk scan, the number of waves used and the
// region bounds, from which the segment's first and last wave w0 .. w1
// follow exactly as in the decode kernel; a segment held by one wave (or an
// empty one) was written by the decode kernel and is skipped.  Wave w keeps
// the partial of its first segment in slot 2 w and of its last in 2 w + 1:
// the segment is the first one of every wave after w0, and of w0 itself
// only when it starts at w0's first chunk.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace {

// Pieces whose partials one step loads at once (every load in flight
// together); a segment with more pieces takes several steps, folded into a
// running (M, L, out).
constexpr int kBatch = 8;

template <int D>
__global__ __launch_bounds__(64) void merge_kernel(SplitParams P) {
  const int seg = blockIdx.x;
  const int b = seg / P.H, g = seg - b * P.H;
  const int32_t c_seq = P.ws_hdr[0];
  const int64_t c_tot = (int64_t)P.H * c_seq;
  const int32_t *s_incl = P.ws_hdr + PKV_HDR_INTS;
  const int cnt = s_incl[b] - (b ? s_incl[b - 1] : 0);
  if (cnt == 0 || c_tot == 0) return;
  const int64_t seg0 = (int64_t)g * c_seq + (s_incl[b] - cnt);
  Regions rg;
  rg.C = c_tot;
  rg.nwe = P.ws_hdr[1];
  rg.nr = P.ws_hdr[2];
  rg.wpr = rg.nwe / rg.nr;
  rg.bounds = reinterpret_cast<const int64_t *>(P.ws_hdr + 4);
  const int w0 = rg.wave_of(seg0), w1 = rg.wave_of(seg0 + cnt - 1);
  const int np = w1 - w0 + 1;
  if (np <= 1) return;
  int64_t lo0, hi0;
  rg.share(w0, lo0, hi0);
  const int first0 = 2 * w0 + (lo0 < seg0 ? 1 : 0);

  const int lane = threadIdx.x, G = P.G;
  const size_t row0 = (size_t)b * P.Hq + (size_t)g * G;
  for (int u = lane; u < G * (D / 4); u += 64) {
    const int h = u / (D / 4), d = 4 * (u % (D / 4));
    float M = -INFINITY, L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i0 = 0; i0 < np; i0 += kBatch) {
      float2 ml[kBatch];
      float4 o[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        // Past the last piece the batch re-reads it and gives it no weight.
        const int i = min(i0 + k, np - 1);
        const size_t r = (size_t)min(i == 0 ? first0 : 2 * (w0 + i), P.nslots - 1) * G + h;
        ml[k] = *reinterpret_cast<const float2 *>(P.ws_ml + 2 * r);
        o[k] = *reinterpret_cast<const float4 *>(P.ws_o + r * D + d);
      }
      float Mb = M;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) Mb = i0 + k < np ? fmaxf(Mb, ml[k].x) : Mb;
      const float fo = fast_exp2(M - Mb);  // 0 on the first step (M = -inf)
      L *= fo;
      acc.x *= fo;
      acc.y *= fo;
      acc.z *= fo;
      acc.w *= fo;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const float f = i0 + k < np ? fast_exp2(ml[k].x - Mb) : 0.f;
        L += ml[k].y * f;
        acc.x += o[k].x * f;
        acc.y += o[k].y * f;
        acc.z += o[k].z * f;
        acc.w += o[k].w * f;
      }
      M = Mb;
    }
    const float inv = 1.f / L;
    *reinterpret_cast<float4 *>(P.out + (row0 + h) * D + d) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
}

}  // namespace

int pkv_launch_merge(const pkv_decode_args &a) {
  const SplitParams p = pkv_split_params(a);
  dim3 grid(a.num_seqs * a.L->num_kv_heads);
  if (a.L->head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(64), 0, reinterpret_cast<hipStream_t>(a.stream), p);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(64), 0, reinterpret_cast<hipStream_t>(a.stream), p);
  return (int)hipGetLastError();
}
