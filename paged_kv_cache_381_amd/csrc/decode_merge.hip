// Split-context merge of the decode kernels' partial results.
//
// A context cut between waves of the balanced split (pkv_device.h) leaves one
// partial per wave: its running maximum m_i (base 2), weight sum l_i and
// unnormalised output o_i.  The whole-context softmax is recovered with
// M = max m_i, L = sum l_i 2^(m_i - M), out = sum o_i 2^(m_i - M) / L, which is
// exact algebra (log-sum-exp), so the result equals a single softmax over all
// tokens.
//
// One workgroup per (sequence, kv head) segment, a thread per 4 output
// columns of a query row (G * D / 4 of them, up to 256 at once: every partial
// of a segment is requested in one round trip after the header's, G <= 8 at
// D = 128).  The schedule header written by
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

constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(SplitParams P) {
  const int seg = blockIdx.x;
  const int b = seg / P.H, g = seg - b * P.H;
  const int32_t *hdr = P.ws_hdr;
  const int32_t *s_incl = hdr + PKV_HDR_INTS;
  // Every header word needed without per-XCD weights is loaded at once (one
  // memory round trip); with them the region bounds are read as well.
  const int32_t c_seq = sload_i32(hdr), nwe = sload_i32(hdr + 1), nr = sload_i32(hdr + 2);
  const int incl = sload_i32(s_incl + b), excl = b ? sload_i32(s_incl + b - 1) : 0;
  const int cnt = incl - excl;
  if (cnt == 0 || c_seq == 0) return;
  const int64_t c_tot = (int64_t)P.H * c_seq;
  const int64_t seg0 = (int64_t)g * c_seq + excl;
  int w0, w1, first0;
  if (nr <= 1) {  // one region [0, c_tot): shares [w C / nwe, (w + 1) C / nwe)
    w0 = (int)(((seg0 + 1) * nwe - 1) / c_tot);
    w1 = (int)(((seg0 + cnt) * nwe - 1) / c_tot);
    first0 = 2 * w0 + ((int64_t)w0 * c_tot / nwe < seg0 ? 1 : 0);
  } else {
    Regions rg;
    rg.C = c_tot;
    rg.nwe = nwe;
    rg.nr = nr;
    rg.wpr = nwe / nr;
    rg.bounds = reinterpret_cast<const int64_t *>(hdr + 4);
    w0 = rg.wave_of(seg0);
    w1 = rg.wave_of(seg0 + cnt - 1);
    int64_t lo0, hi0;
    rg.share(w0, lo0, hi0);
    first0 = 2 * w0 + (lo0 < seg0 ? 1 : 0);
  }
  const int np = w1 - w0 + 1;
  if (np <= 1) return;

  const int tid = threadIdx.x, G = P.G;
  const size_t row0 = (size_t)b * P.Hq + (size_t)g * G;
  for (int u = tid; u < G * (D / 4); u += kMergeThreads) {
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
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kMergeThreads), 0, reinterpret_cast<hipStream_t>(a.stream), p);
  else
    hipLaunchKernelGGL(merge_kernel<64>, grid, dim3(kMergeThreads), 0, reinterpret_cast<hipStream_t>(a.stream), p);
  return (int)hipGetLastError();
}
