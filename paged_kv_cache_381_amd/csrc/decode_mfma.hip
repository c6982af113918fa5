// PagedAttention decode, matrix-core kernel (bf16 KV, grouped-query heads).
//
// What it computes [KV Cache 工程学 §15.5; 新一代 KV Cache 管理 §8.1]: for a
// sequence b and its query heads h of kv group g, the new token's query is
// dotted with the K of every cached token, found by reading block-table entry
// j/16 and slot j%16; a softmax over the whole context weights the cached V.
// The context is visited 32 tokens at a time with a running maximum and sum
// (online softmax), so the softmax stays global even though the data arrive
// block by block (the per-page softmax of the vendor article
// [PagedAttention：大模型KV Cache内存管理革新 §3.2] is not used).
//
// Work split.  Persistent waves each take one equal, contiguous share of the
// batch's 32-token chunks (pkv_device.h, "Balanced split"): the mix of
// context lengths does not leave a tail of long sequences running alone.
// Within its share a wave walks (sequence, kv head) segments in order; a
// segment it holds entirely is normalised and stored, a segment cut by a share
// boundary leaves a partial (m, l, o) for the merge kernel.
//
// gfx950 mapping.  The G query heads of a group share every K and V tile, so
// the group-by-block products are small dense contractions and run on
// v_mfma_f32_16x16x32_bf16, with the G heads padded to 16 columns:
//   S^T[32 tokens x 16 heads] = K[32 x D] . Q^T[D x 16]   (two 16-row MFMAs)
//   O^T[D x 16 heads]        += V^T[D x 32] . P^T[32 x 16] (D/16 MFMAs)
// A chunk is two 16-token blocks.  Lane (c = lane%16, j = lane/16) receives S
// for head c and tokens {8(j%2) + 0..3} (first MFMA) and {8(j%2) + 4..7}
// (second MFMA) of block j/2 -- exactly the eight token slots it must hand to
// the PV MFMA, whose V^T operand for lane (d, j) is then 16 contiguous bytes
// of the [D][16] V tile (tokens 8(j%2)..+7 of block j/2).  No cross-lane
// shuffle sits between the two contractions; the softmax needs only two
// xor-shuffles per chunk (max over the four lane groups).  Each lane holds the
// 8-element slices of the group's query rows that its B operand needs, read
// straight from memory once per segment: the whole group shares them through
// the MFMA, and nothing else in the wave would reuse an LDS copy.
//
// Memory pipeline.  Block ids and lengths are scalar loads issued one chunk
// ahead; chunk c+1's K is requested as soon as chunk c's score MFMAs have
// consumed the K registers and its V once the PV MFMAs have consumed V, so a
// wave always has a chunk of loads in flight through its own math.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace {

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Zero the bf16 elements of u whose index is >= nvalid (0..8).
__device__ __forceinline__ uint4 keep_first(uint4 u, int nvalid) {
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t mask = (2 * k + 1 < nvalid) ? 0xffffffffu : (2 * k < nvalid ? 0x0000ffffu : 0u);
    w[k] &= mask;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

#ifndef PKV_MFMA_MIN_WAVES_PER_SIMD
#define PKV_MFMA_MIN_WAVES_PER_SIMD 1
#endif

template <int D, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(PKV_MFMA_MIN_WAVES_PER_SIMD)))
void decode_mfma_kernel(SplitParams P) {
  constexpr int NKK = D / 32;  // score MFMAs per 16-row token set
  constexpr int NNN = D / 16;  // PV MFMAs
  constexpr int TILE = 16 * D;
  extern __shared__ __align__(16) int32_t s_incl[];  // [B] inclusive chunk scan, then [W] scratch
  int32_t *s_wave = s_incl + P.B;

  const int lane = threadIdx.x & 63;
  const int H = P.H, G = P.G;
  Share sh;
  if (!split_begin<W, D>(P, s_incl, s_wave, sh)) return;
  const int64_t lo = sh.lo, hi = sh.hi;
  Cursor cur = sh.first();

  const int r16 = lane & 15, grp = lane >> 4;
  // Row r16 of the score MFMAs holds a token of block (r16 >> 3); see header.
  const int ksel = r16 >> 3;
  const int ktx = ((r16 >> 2) & 1) * 8 + (r16 & 3);
  const int vsel = grp >> 1, vhalf = grp & 1;

  const uint16_t *kpool = reinterpret_cast<const uint16_t *>(P.k_pool);
  const uint16_t *vpool = reinterpret_cast<const uint16_t *>(P.v_pool);
  const uint16_t *qbase = reinterpret_cast<const uint16_t *>(P.q);
  bf16x8_t qb[NKK];
  uint4 ax[NKK], ay[NKK], va[NNN];

  auto load_q = [&](const Cursor &c) {
    // Columns G..15 of the B operand are zero; their lanes read row G-1 (in
    // bounds) and discard it.
    const int h = min(r16, G - 1);
    const uint4 *qr = reinterpret_cast<const uint4 *>(qbase + ((size_t)c.b * P.Hq + (size_t)c.g * G + h) * D);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint4 u = qr[4 * kk + grp];
      qb[kk] = as_bf16x8(r16 < G ? u : make_uint4(0, 0, 0, 0));
    }
  };
  auto load_k = [&](int g, int pa, int pb) {
    const uint4 *kt = reinterpret_cast<const uint4 *>(kpool + ((size_t)(ksel ? pb : pa) * H + g) * TILE);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int c = 4 * kk + grp;
      ax[kk] = kt[c * 16 + ktx];
      ay[kk] = kt[c * 16 + ktx + 4];
    }
  };
  auto load_v = [&](int g, int pa, int pb) {
    const uint4 *vt = reinterpret_cast<const uint4 *>(vpool + ((size_t)(vsel ? pb : pa) * H + g) * TILE);
#pragma unroll
    for (int nn = 0; nn < NNN; ++nn) va[nn] = vt[2 * (16 * nn + r16) + vhalf];
  };

  int pa, pb;
  sh.blocks(cur, pa, pb);
  load_q(cur);
  load_k(cur.g, pa, pb);
  load_v(cur.g, pa, pb);
  Cursor nxt = cur;
  int npa = 0, npb = 0;
  if (lo + 1 < hi) {
    nxt = sh.next(cur);
    sh.blocks(nxt, npa, npb);
  }

  f32x4_t o[NNN];
#pragma unroll
  for (int nn = 0; nn < NNN; ++nn) o[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  for (int64_t x = lo; x < hi; ++x) {
    f32x4_t sx = {0.f, 0.f, 0.f, 0.f}, sy = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      sx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ax[kk]), qb[kk], sx, 0, 0, 0);
      sy = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ay[kk]), qb[kk], sy, 0, 0, 0);
    }
    const bool more = x + 1 < hi;
    const bool seg_end = !more || nxt.j == 0;
    if (more) {
      if (nxt.j == 0) load_q(nxt);  // the score MFMAs above have consumed qb
      load_k(nxt.g, npa, npb);
    }

    const int n = cur.n;
    const int tok0 = 32 * cur.j;
    const int tb = tok0 + 16 * (grp >> 1) + 8 * (grp & 1);
    float s[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = (tb + r < n) ? sx[r] * P.scale_log2 : -INFINITY;
      s[4 + r] = (tb + 4 + r < n) ? sy[r] * P.scale_log2 : -INFINITY;
    }
    float cmax = s[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) cmax = fmaxf(cmax, s[r]);
    cmax = rows_max4(cmax);
    const float mnew = fmaxf(m, cmax);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    bf16x8_t pv;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const __bf16 pr = (__bf16)fast_exp2(s[r] - mnew);
      pv[r] = pr;
      psum += (float)pr;  // the PV numerator uses the rounded weights too
    }
    l = l * alpha + psum;
#pragma unroll
    for (int nn = 0; nn < NNN; ++nn) o[nn] *= alpha;
    if (tok0 + 32 > n) {  // slots past the context may hold anything, NaN included
      const int nvalid = min(max(n - tb, 0), 8);  // tb is this lane's first V token
#pragma unroll
      for (int nn = 0; nn < NNN; ++nn) va[nn] = keep_first(va[nn], nvalid);
    }
#pragma unroll
    for (int nn = 0; nn < NNN; ++nn) o[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va[nn]), pv, o[nn], 0, 0, 0);
    if (more) load_v(nxt.g, npa, npb);

    if (seg_end) {
      const float lsum = rows_sum4(l);
      const bool whole = sh.whole(cur);
      if (r16 < G) {
        const size_t row = (size_t)cur.b * P.Hq + (size_t)cur.g * G + r16;
        if (whole) {
          const float inv = 1.f / lsum;
          float *dst = P.out + row * D + 4 * grp;
#pragma unroll
          for (int nn = 0; nn < NNN; ++nn)
            *reinterpret_cast<float4 *>(dst + 16 * nn) =
                make_float4(o[nn][0] * inv, o[nn][1] * inv, o[nn][2] * inv, o[nn][3] * inv);
        } else {
          const size_t slot = row * P.maxp + sh.piece(cur, P.maxp);
          float *dst = P.ws_o + slot * D + 4 * grp;
#pragma unroll
          for (int nn = 0; nn < NNN; ++nn)
            *reinterpret_cast<float4 *>(dst + 16 * nn) = make_float4(o[nn][0], o[nn][1], o[nn][2], o[nn][3]);
          if (grp == 0) *reinterpret_cast<float2 *>(P.ws_ml + 2 * slot) = make_float2(m, lsum);
        }
      }
#pragma unroll
      for (int nn = 0; nn < NNN; ++nn) o[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m = -INFINITY;
      l = 0.f;
    }

    if (more) {
      cur = nxt;
      if (x + 2 < hi) {
        nxt = sh.next(cur);
        sh.blocks(nxt, npa, npb);
      }
    }
  }
}

#ifndef PKV_MFMA_WAVES
#define PKV_MFMA_WAVES 4
#endif
constexpr int kWaves = PKV_MFMA_WAVES;

template <int D>
int launch(const pkv_decode_args &a, const SplitParams &p) {
  auto kern = decode_mfma_kernel<D, kWaves>;
  const size_t lds = pkv_split_lds_bytes(a.num_seqs, kWaves);
  int nwg = 0;
  if (int rc = pkv_split_grid(reinterpret_cast<const void *>(kern), 64 * kWaves, lds, a, &nwg)) return rc;
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(64 * kWaves), lds, reinterpret_cast<hipStream_t>(a.stream), p);
  return (int)hipGetLastError();
}

}  // namespace

int pkv_launch_decode_mfma(const pkv_decode_args &a) {
  const SplitParams p = pkv_split_params(a);
  return a.L->head_dim == 128 ? launch<128>(a, p) : launch<64>(a, p);
}
