// Paged prefill: causal attention of a sequence's new tokens over its paged
// cache, on the matrix cores (bf16 or int8 cache).
//
// What it computes [KV Cache 工程学 §15.1: a prompt is a causal i x i
// attention; §15.6 and 新一代 KV Cache 管理 §8.3: a cached prefix is not
// prefilled again]: sequence b holds ctx_b tokens in its table, the last
// nq_b of them new (their K/V already stored by paged_kv_append).  New token t
// sits at position p_b + t, p_b = ctx_b - nq_b, and attends to positions
// 0 .. p_b + t -- the cached prefix and the new tokens up to itself.
//
// gfx950 mapping.  The decode kernel's contractions are reused with the
// padding gone: a wave takes 16 query columns, TQ = 16 / G consecutive new
// tokens times the G query heads of one kv head g, so every column of
//   S^T[32 keys x 16 columns] = K[32 x D] . Q^T[D x 16]
//   O^T[D x 16 columns]      += V^T[D x 32] . P^T[32 x 16]
// is a real query row.  The operand layouts, the lane holding 8 keys of one
// column between the two products and the online softmax per column are the
// decode kernel's; the causal limit differs per column and masks scores per
// lane.  A wave walks keys 0 .. its last token's position in 32-key chunks
// (two blocks through the table), with NB chunks of K/V in registers, every
// load issued on every path so that the memory-counter waits stay exact.
// Tiles of one (sequence, kv head) that run longest (the last tokens) are
// dispatched first.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace {

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Eight int8 codes, widened exactly to bf16.
__device__ __forceinline__ bf16x8_t as_bf16x8(uint2 u) {
  bf16x8_t r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    r[k] = (__bf16)(float)(int8_t)(u.x >> (8 * k));
    r[4 + k] = (__bf16)(float)(int8_t)(u.y >> (8 * k));
  }
  return r;
}

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

constexpr float kSlack = 8.0f;  // headroom of the running maximum (base 2)

template <int D, int NB, bool I8, int CT>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(PrefillParams P) {
  constexpr int NKK = D / 32;
  constexpr int NNN = D / 16;
  constexpr int TB = I8 ? 16 * D + 64 : 32 * D;
  constexpr int NKU = I8 ? NKK / 2 : NKK;
  using VUnit = std::conditional_t<I8, uint2, uint4>;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int b = blockIdx.z, g = blockIdx.y;
  const int G = P.G, TQ = 16 / G;
  const int q0 = sload_i32(P.qstart + b);
  const int n = clamp_len(sload_i32(P.ctx + b), P.max_blocks, P.max_ctx);
  // A sequence claiming more new tokens than it holds keeps its last n.
  const int nq = min(sload_i32(P.qstart + b + 1) - q0, n);
  const int ntile = (nq + TQ - 1) / TQ;
  // The wave's CT column tiles, longest first; tiles run longest first too.
  const int t_first = ntile - 1 - (int)(blockIdx.x * 4 + w) * CT;
  if (t_first < 0) return;
  const int p0 = n - nq;  // position of new token 0
  const int kend = p0 + min(t_first * TQ + TQ, nq);  // keys the wave's last token sees
  const int nch = (kend + 31) >> 5;

  // The earliest column's causal limit: chunks up to it are open to all.
  const int pos_min = p0 + max(t_first - CT + 1, 0) * TQ;

  const int r16 = lane & 15, grp = lane >> 4;
  // Column r16 of tile t: token t*TQ + r16/G, head r16%G of group g.
  // Columns past TQ*G or past the last new token, and tiles before the
  // first, repeat a real column and store nothing.
  const int cc = min(r16, TQ * G - 1);
  int pos[CT];
  bool store_col[CT];
  size_t qrow[CT];
#pragma unroll
  for (int s = 0; s < CT; ++s) {
    const int t = t_first - s;
    const int tt = t < 0 ? t_first : t;
    const int tlast = min(tt * TQ + TQ, nq) - 1;
    const int tcol = min(tt * TQ + cc / G, tlast);
    store_col[s] = t >= 0 && r16 < TQ * G && tt * TQ + r16 / G <= tlast;
    pos[s] = p0 + tcol;  // the column's causal limit (inclusive)
    qrow[s] = (size_t)(q0 + tcol) * P.Hq + (size_t)g * G + cc % G;
  }

  const int ksel = r16 >> 3;
  const int ktx = ((r16 >> 2) & 1) * 8 + (r16 & 3);
  const int vsel = grp >> 1, vhalf = grp & 1;
  auto kgroup = [&](int kk) { return I8 ? 8 * (kk >> 1) + 2 * grp + (kk & 1) : 4 * kk + grp; };
  const uint8_t *kpool = reinterpret_cast<const uint8_t *>(P.k_pool);
  const uint8_t *vpool = reinterpret_cast<const uint8_t *>(P.v_pool);
  const int32_t *trow = P.tables + (size_t)b * P.max_blocks;
  const int H = P.H;

  // The query slices stay in registers for the whole walk.
  bf16x8_t qb[CT][NKK];
#pragma unroll
  for (int s = 0; s < CT; ++s) {
    const uint4 *qr = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(P.q) + qrow[s] * D);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qb[s][kk] = as_bf16x8(qr[kgroup(kk)]);
  }

  int cj[NB], pa[NB], pb[NB];
  uint4 ax[NB][NKU], ay[NB][NKU];
  VUnit va[NB][NNN];
  float4 ksc[NB][2], vsc[NB][2];

  auto locate = [&](int i, int c) {
    cj[i] = c;
    pa[i] = clamp_block(sload_i32(trow + 2 * c), P.num_blocks);
    const int b2 = clamp_block(sload_i32(trow + min(2 * c + 1, P.max_blocks - 1)), P.num_blocks);
    pb[i] = 32 * c + 16 < kend ? b2 : pa[i];
  };
  auto same_as = [&](int to, int from) {
    cj[to] = cj[from];
    pa[to] = pa[from];
    pb[to] = pb[from];
  };
  auto issue = [&](auto bi) {
    constexpr int I = decltype(bi)::value;
    const uint4 *kt = reinterpret_cast<const uint4 *>(kpool + ((size_t)(ksel ? pb[I] : pa[I]) * H + g) * TB);
#pragma unroll
    for (int ku = 0; ku < NKU; ++ku) {
      const int cu = 4 * ku + grp;
      ax[I][ku] = kt[cu * 16 + ktx];
      ay[I][ku] = kt[cu * 16 + ktx + 4];
    }
    if constexpr (I8) {
      const float4 *sc = reinterpret_cast<const float4 *>(kpool + ((size_t)(vsel ? pb[I] : pa[I]) * H + g) * TB +
                                                          16 * D + 32 * vhalf);
      ksc[I][0] = sc[0];
      ksc[I][1] = sc[1];
    }
  };
  auto issue_v = [&](auto bi) {
    constexpr int I = decltype(bi)::value;
    const uint8_t *vt = vpool + ((size_t)(vsel ? pb[I] : pa[I]) * H + g) * TB;
    if constexpr (I8) {
#pragma unroll
      for (int nn = 0; nn < NNN; ++nn) va[I][nn] = *reinterpret_cast<const uint2 *>(vt + (16 * nn + r16) * 16 + 8 * vhalf);
      const float4 *sc = reinterpret_cast<const float4 *>(vt + 16 * D + 32 * vhalf);
      vsc[I][0] = sc[0];
      vsc[I][1] = sc[1];
    } else {
      const uint4 *u = reinterpret_cast<const uint4 *>(vt);
#pragma unroll
      for (int nn = 0; nn < NNN; ++nn) va[I][nn] = u[2 * (16 * nn + r16) + vhalf];
    }
  };

  f32x4_t o[CT][NNN];
  float m[CT], l[CT];
#pragma unroll
  for (int s = 0; s < CT; ++s) {
#pragma unroll
    for (int nn = 0; nn < NNN; ++nn) o[s][nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m[s] = -INFINITY;
    l[s] = 0.f;
  }

  locate(0, 0);
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    ((Is == 0 ? (void)0 : (Is < nch ? locate(Is, Is) : same_as(Is, Is - 1))), ...);
  }(std::make_integer_sequence<int, NB>{});
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    ((Is < NB - 1 ? (issue(std::integral_constant<int, Is>{}), __builtin_amdgcn_sched_barrier(0),
                     issue_v(std::integral_constant<int, Is>{}), __builtin_amdgcn_sched_barrier(0))
                  : (void)0),
     ...);
  }(std::make_integer_sequence<int, NB>{});

  int x = 0;
  auto step = [&](auto bi) {
    constexpr int I = decltype(bi)::value;
    constexpr int J = (I + NB - 1) % NB;
    f32x4_t sx[CT], sy[CT];
#pragma unroll
    for (int s = 0; s < CT; ++s) sx[s] = sy[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8_t kx, ky;
      if constexpr (I8) {
        const uint4 ux = ax[I][kk >> 1], uy = ay[I][kk >> 1];
        kx = as_bf16x8((kk & 1) ? make_uint2(ux.z, ux.w) : make_uint2(ux.x, ux.y));
        ky = as_bf16x8((kk & 1) ? make_uint2(uy.z, uy.w) : make_uint2(uy.x, uy.y));
      } else {
        kx = as_bf16x8(ax[I][kk]);
        ky = as_bf16x8(ay[I][kk]);
      }
#pragma unroll
      for (int s = 0; s < CT; ++s) {
        sx[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kx, qb[s][kk], sx[s], 0, 0, 0);
        sy[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ky, qb[s][kk], sy[s], 0, 0, 0);
      }
    }
    if (x + NB - 1 >= nch) same_as(J, I);
    issue(std::integral_constant<int, J>{});

    // Keys of this lane: 8 consecutive positions from tb.  Past the walk's
    // end (x >= nch) nothing is counted.
    const bool real = x < nch;
    const int tb = 32 * cj[I] + 16 * vsel + 8 * vhalf;
    float ks[8], vs[8];
    if constexpr (I8) {
      ks[0] = ksc[I][0].x; ks[1] = ksc[I][0].y; ks[2] = ksc[I][0].z; ks[3] = ksc[I][0].w;
      ks[4] = ksc[I][1].x; ks[5] = ksc[I][1].y; ks[6] = ksc[I][1].z; ks[7] = ksc[I][1].w;
      vs[0] = vsc[I][0].x; vs[1] = vsc[I][0].y; vs[2] = vsc[I][0].z; vs[3] = vsc[I][0].w;
      vs[4] = vsc[I][1].x; vs[5] = vsc[I][1].y; vs[6] = vsc[I][1].z; vs[7] = vsc[I][1].w;
    }
    bf16x8_t pv[CT];
    // A chunk below every column's causal limit needs no mask (most chunks of
    // a long prefix): the running maximum is taken on raw scores (scale > 0)
    // and each weight is one fma and one exp2.
    const bool open = !I8 && real && 32 * cj[I] + 31 <= pos_min && P.scale_log2 > 0.f;
    if (open) {
#pragma unroll
      for (int s = 0; s < CT; ++s) {
        float cmax = fmaxf(fmaxf(sx[s][0], sx[s][1]), fmaxf(sx[s][2], sx[s][3]));
        cmax = fmaxf(cmax, fmaxf(fmaxf(sy[s][0], sy[s][1]), fmaxf(sy[s][2], sy[s][3])));
        cmax = rows_max4_swap(cmax) * P.scale_log2;
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(cmax > m[s] + kSlack) != 0, 0)) {
          const float mnew = fmaxf(m[s], cmax);
          const float alpha = fast_exp2(m[s] - mnew);
          m[s] = mnew;
          l[s] *= alpha;
#pragma unroll
          for (int nn = 0; nn < NNN; ++nn) o[s][nn] *= alpha;
        }
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const __bf16 px = (__bf16)fast_exp2(__builtin_fmaf(sx[s][r], P.scale_log2, -m[s]));
          const __bf16 py = (__bf16)fast_exp2(__builtin_fmaf(sy[s][r], P.scale_log2, -m[s]));
          pv[s][r] = px;
          pv[s][4 + r] = py;
          psum += (float)px + (float)py;
        }
        l[s] += psum;
      }
    }
#pragma unroll
    for (int s = 0; s < CT && !open; ++s) {
      const int lim = real ? pos[s] : -1;
      float sc[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float kx = I8 ? ks[r] : 1.f, ky = I8 ? ks[4 + r] : 1.f;
        sc[r] = (tb + r <= lim) ? sx[s][r] * kx * P.scale_log2 : -INFINITY;
        sc[4 + r] = (tb + 4 + r <= lim) ? sy[s][r] * ky * P.scale_log2 : -INFINITY;
      }
      float cmax = sc[0];
#pragma unroll
      for (int r = 1; r < 8; ++r) cmax = fmaxf(cmax, sc[r]);
      cmax = rows_max4_swap(cmax);
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(cmax > m[s] + kSlack) != 0, 0)) {
        const float mnew = fmaxf(m[s], cmax);
        const float alpha = fast_exp2(m[s] - mnew);
        m[s] = mnew;
        l[s] *= alpha;
#pragma unroll
        for (int nn = 0; nn < NNN; ++nn) o[s][nn] *= alpha;
      }
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if constexpr (I8) {
          const float e = fast_exp2(sc[r] - m[s]);
          psum += e;
          pv[s][r] = (__bf16)((tb + r <= lim) ? e * vs[r] : 0.f);  // scales past the context may be NaN
        } else {
          const __bf16 pr = (__bf16)fast_exp2(sc[r] - m[s]);
          pv[s][r] = pr;
          psum += (float)pr;
        }
      }
      l[s] += psum;
    }
    if constexpr (!I8) {
      // Keys at or past the walk's end may be unwritten (NaN); a zero weight
      // alone would not cancel them.
      const int nvalid = real ? min(max(kend - tb, 0), 8) : 0;
      if (nvalid < 8) {
#pragma unroll
        for (int nn = 0; nn < NNN; ++nn) va[I][nn] = keep_first(va[I][nn], nvalid);
      }
    }
#pragma unroll
    for (int nn = 0; nn < NNN; ++nn) {
      const bf16x8_t vop = as_bf16x8(va[I][nn]);
#pragma unroll
      for (int s = 0; s < CT; ++s) o[s][nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pv[s], o[s][nn], 0, 0, 0);
    }
    issue_v(std::integral_constant<int, J>{});
    if (x + NB < nch) locate(I, x + NB);
    ++x;
  };
  while (x < nch) {
    [&]<int... Is>(std::integer_sequence<int, Is...>) {
      (step(std::integral_constant<int, Is>{}), ...);
    }(std::make_integer_sequence<int, NB>{});
  }

#pragma unroll
  for (int s = 0; s < CT; ++s) {
    const float lsum = rows_sum4(l[s]);
    if (store_col[s]) {
      const float inv = 1.f / lsum;
      float *dst = P.out + qrow[s] * D + 4 * grp;
#pragma unroll
      for (int nn = 0; nn < NNN; ++nn)
        *reinterpret_cast<float4 *>(dst + 16 * nn) =
            make_float4(o[s][nn][0] * inv, o[s][nn][1] * inv, o[s][nn][2] * inv, o[s][nn][3] * inv);
    }
  }
}

#ifndef PKV_PREFILL_NBUF
#define PKV_PREFILL_NBUF 2
#endif
#ifndef PKV_PREFILL_NBUF_I8
#define PKV_PREFILL_NBUF_I8 4
#endif

// Column tiles (16 query columns each) per wave: the K and V operands of a
// chunk serve all of them, so each byte read from L2 feeds CT x the math.
#ifndef PKV_PREFILL_CT
#define PKV_PREFILL_CT 2
#endif

template <int D, bool I8>
int launch(const pkv_prefill_args &a, const PrefillParams &p) {
  constexpr int CT = PKV_PREFILL_CT;
  auto kern = prefill_mfma_kernel<D, I8 ? PKV_PREFILL_NBUF_I8 : PKV_PREFILL_NBUF, I8, CT>;
  const int tq = 16 / p.G;
  const int tiles = (a.max_query_len + tq - 1) / tq;
  const int waves = (tiles + CT - 1) / CT;
  const dim3 grid((unsigned)((waves + 3) / 4), (unsigned)p.H, (unsigned)a.num_seqs);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, reinterpret_cast<hipStream_t>(a.stream), p);
  return (int)hipGetLastError();
}

}  // namespace

int pkv_launch_prefill_mfma(const pkv_prefill_args &a) {
  PrefillParams p;
  p.out = a.out;
  p.q = a.q;
  p.k_pool = a.k_pool;
  p.v_pool = a.v_pool;
  p.tables = a.tables;
  p.ctx = a.ctx;
  p.qstart = a.qstart;
  p.num_blocks = a.L->num_blocks;
  p.H = a.L->num_kv_heads;
  p.Hq = a.num_q_heads;
  p.G = a.num_q_heads / a.L->num_kv_heads;
  p.max_blocks = a.max_blocks;
  p.max_ctx = a.max_ctx;
  p.scale_log2 = a.scale_log2;
  if (a.L->kv_dtype == PKV_INT8) return a.L->head_dim == 128 ? launch<128, true>(a, p) : launch<64, true>(a, p);
  return a.L->head_dim == 128 ? launch<128, false>(a, p) : launch<64, false>(a, p);
}
