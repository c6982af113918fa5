// PagedAttention decode, wavefront-reduction kernel (bf16 or fp32 KV, any
// group size up to 16).
//
// Same computation as the matrix-core kernel [KV Cache 工程学 §15.5;
// 新一代 KV Cache 管理 §8.1]: scores of the new token's query against every
// cached key, fetched through the block table, a softmax over the whole
// context kept as a running maximum and sum, and the weighted sum of V.  It
// serves multi-head attention (one query head per kv head, where a group
// product is a matrix-vector product and gains nothing from matrix cores) and
// float32 caches.  Work is split over persistent waves exactly as in the
// matrix-core kernel (pkv_device.h, "Balanced split").
//
// gfx950 mapping, per wave and 32-token chunk (two 16-token blocks; each
// block is one 16*D-element tile of K and one of V, read as 16-byte units
// u = 64 i + lane, fully coalesced):
//   K tile [D/X][16][X]: lane holds token lane%16 for d-chunks 4i + lane/16,
//     so a score is an in-lane dot over D/4 elements plus a two-step
//     cross-row reduction (lanes l, l^16, l^32, l^48);
//   the chunk maximum is a DPP all-reduce inside a 16-lane row;
//   V tile [D][16]: lane holds X consecutive tokens of one d, so the weights
//     of those tokens are read back from a per-wave LDS line and the lane
//     accumulates out[d] directly; lanes sharing a d are folded with one or
//     two DPP steps when a segment ends.
// The query rows of the group are staged once per segment in the wave's own
// LDS slice as float: every lane needs every element of its d-chunks for all
// G heads, so they are read from LDS (or, when they fit, kept in registers)
// instead of being fetched again per token.
//
// Memory pipeline as in the matrix-core kernel: block ids are scalar loads one
// chunk ahead, chunk c+1's K is requested once chunk c's scores are done and
// its V once chunk c's V has been accumulated.
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

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Per-wave LDS floats: the group's query rows and one chunk of weights.
template <int D, int GP>
constexpr int wave_lds_floats() {
  return GP * D + GP * 32;
}

template <typename E, int D, int GP, int W, bool NT>
__global__ __launch_bounds__(64 * W) void decode_valu_kernel(SplitParams P) {
  constexpr int ES = sizeof(E);
  constexpr int X = 16 / ES;       // elements per 16-byte unit
  constexpr int NL = D * ES / 64;  // units per lane per tile (a tile is D*ES units)
  constexpr int TILE = 16 * D;
  constexpr int QN = GP * D / 64;  // query elements each lane stages
  constexpr bool QREG = GP * NL * X <= 64;
  extern __shared__ __align__(16) int32_t s_lds[];  // chunk scan, lengths, wave totals, then per-wave slices
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float *q_lds = reinterpret_cast<float *>(s_lds + pkv_split_lds_ints(P.B, W)) + w * wave_lds_floats<D, GP>();
  float *p_lds = q_lds + GP * D;  // [GP][32]

  Share sh;
  if (!split_begin<W, D>(P, s_lds, sh)) return;
  const int64_t lo = sh.lo, hi = sh.hi;
  const int H = P.H, G = P.G;
  const int tok = lane & 15, row = lane >> 4;
  const int vpart = lane % ES;  // which X-token run of a V row this lane reads

  const E *kpool = reinterpret_cast<const E *>(P.k_pool);
  const E *vpool = reinterpret_cast<const E *>(P.v_pool);
  uint4 ku[2][NL], vu[2][NL];
  float qn[QN];  // the next segment's query elements, in flight
  float qr[QREG ? GP : 1][QREG ? NL : 1][QREG ? X : 1];

  auto fetch_q = [&](const Cursor &c) {
    const size_t qoff = ((size_t)c.b * P.Hq + (size_t)c.g * G) * D;
#pragma unroll
    for (int k = 0; k < QN; ++k) {
      const int i = 64 * k + lane;
      qn[k] = (i / D) < G ? load_elem<E>(P.q, qoff + i) : 0.f;
    }
  };
  auto stage_q = [&]() {  // qn -> the wave's LDS slice (and registers)
#pragma unroll
    for (int k = 0; k < QN; ++k) q_lds[64 * k + lane] = qn[k];
    wave_sync_lds();
    if constexpr (QREG) {
#pragma unroll
      for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
          for (int e = 0; e < X; ++e) qr[h][i][e] = q_lds[h * D + (4 * i + row) * X + e];
    }
  };
  auto qval = [&](int h, int i, int e) -> float {
    if constexpr (QREG)
      return qr[h][i][e];
    else
      return q_lds[h * D + (4 * i + row) * X + e];
  };
  auto load_k = [&](int g, int pa, int pb) {
    const uint4 *ka = reinterpret_cast<const uint4 *>(kpool + ((size_t)pa * H + g) * TILE);
    const uint4 *kb = reinterpret_cast<const uint4 *>(kpool + ((size_t)pb * H + g) * TILE);
#pragma unroll
    for (int i = 0; i < NL; ++i) ku[0][i] = load_u4<NT>(ka + 64 * i + lane);
#pragma unroll
    for (int i = 0; i < NL; ++i) ku[1][i] = load_u4<NT>(kb + 64 * i + lane);
  };
  auto load_v = [&](int g, int pa, int pb) {
    const uint4 *va = reinterpret_cast<const uint4 *>(vpool + ((size_t)pa * H + g) * TILE);
    const uint4 *vb = reinterpret_cast<const uint4 *>(vpool + ((size_t)pb * H + g) * TILE);
#pragma unroll
    for (int i = 0; i < NL; ++i) vu[0][i] = load_u4<NT>(va + 64 * i + lane);
#pragma unroll
    for (int i = 0; i < NL; ++i) vu[1][i] = load_u4<NT>(vb + 64 * i + lane);
  };

  Cursor cur = sh.first();
  int pa, pb;
  sh.blocks(cur, pa, pb);
  fetch_q(cur);
  load_k(cur.g, pa, pb);
  load_v(cur.g, pa, pb);
  stage_q();
  Cursor nxt = cur;
  int npa = 0, npb = 0;
  if (lo + 1 < hi) {
    nxt = sh.next(cur);
    sh.blocks(nxt, npa, npb);
  }

  float m[GP], lsum[GP], acc[GP][NL];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i) acc[h][i] = 0.f;
  }

  for (int64_t x = lo; x < hi; ++x) {
    const int n = cur.n;
    const int tok0 = 32 * cur.j;
    // Scores of the chunk's 32 tokens: this lane's token in each block.
    float s[2][GP];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk)
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < NL; ++i)
#pragma unroll
          for (int e = 0; e < X; ++e) d += qval(h, i, e) * unit_elem<E>(ku[bk][i], e);
        d = rows_sum4(d);
        s[bk][h] = (tok0 + 16 * bk + tok < n) ? d * P.scale_log2 : -INFINITY;
      }

    const bool more = x + 1 < hi;
    const bool new_seg = more && nxt.j == 0;
    if (more) {
      if (new_seg) fetch_q(nxt);
      load_k(nxt.g, npa, npb);
    }

    float p[2][GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const float mnew = fmaxf(m[h], row_max16(fmaxf(s[0][h], s[1][h])));
      const float alpha = fast_exp2(m[h] - mnew);
      m[h] = mnew;
      p[0][h] = fast_exp2(s[0][h] - mnew);
      p[1][h] = fast_exp2(s[1][h] - mnew);
      lsum[h] = lsum[h] * alpha + p[0][h] + p[1][h];
#pragma unroll
      for (int i = 0; i < NL; ++i) acc[h][i] *= alpha;
    }
    if (row == 0) {
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        p_lds[h * 32 + tok] = p[0][h];
        p_lds[h * 32 + 16 + tok] = p[1][h];
      }
    }
    wave_sync_lds();
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      const int vtok0 = tok0 + 16 * bk + vpart * X;
      const int nvalid = min(max(n - vtok0, 0), X);
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        float pw[X];
#pragma unroll
        for (int e = 0; e < X; ++e) pw[e] = p_lds[h * 32 + 16 * bk + vpart * X + e];
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          float a = acc[h][i];
#pragma unroll
          for (int e = 0; e < X; ++e) {
            const float v = unit_elem<E>(vu[bk][i], e);
            a += (e < nvalid) ? pw[e] * v : 0.f;  // select: a NaN past the end must not leak
          }
          acc[h][i] = a;
        }
      }
    }
    if (more) load_v(nxt.g, npa, npb);
    wave_sync_lds();  // p_lds and q_lds reads of this chunk are done

    if (!more || new_seg) {
      // Lanes sharing a d differ in their low log2(ES) bits.
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        lsum[h] = row_sum16(lsum[h]);
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          acc[h][i] += dpp<PKV_DPP_XOR1>(acc[h][i]);
          if constexpr (ES == 4) acc[h][i] += dpp<PKV_DPP_XOR2>(acc[h][i]);
        }
      }
      const bool whole = sh.whole(cur);
      const int pslot = sh.slot(cur, P.nslots);

#pragma unroll
      for (int h = 0; h < GP; ++h) {
        if (h >= G) continue;
        const size_t rowq = (size_t)cur.b * P.Hq + (size_t)cur.g * G + h;
        if (whole) {
          const float inv = 1.f / lsum[h];
          if (vpart == 0) {
#pragma unroll
            for (int i = 0; i < NL; ++i) P.out[rowq * D + (64 * i + lane) / ES] = acc[h][i] * inv;
          }
        } else {
          const size_t slot = (size_t)pslot * G + h;
          if (vpart == 0) {
#pragma unroll
            for (int i = 0; i < NL; ++i) P.ws_o[slot * D + (64 * i + lane) / ES] = acc[h][i];
          }
          if (lane == 0) *reinterpret_cast<float2 *>(P.ws_ml + 2 * slot) = make_float2(m[h], lsum[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        m[h] = -INFINITY;
        lsum[h] = 0.f;
#pragma unroll
        for (int i = 0; i < NL; ++i) acc[h][i] = 0.f;
      }
    }
    if (more) {
      if (new_seg) stage_q();
      cur = nxt;
      if (x + 2 < hi) {
        nxt = sh.next(cur);
        sh.blocks(nxt, npa, npb);
      }
    }
  }
}

constexpr int kWaves = 4;

template <typename E, int D, int GP>
int launch(const pkv_decode_args &a, const SplitParams &p) {
  auto kern = a.streaming ? decode_valu_kernel<E, D, GP, kWaves, true> : decode_valu_kernel<E, D, GP, kWaves, false>;
  const size_t lds = pkv_split_lds_bytes(a.num_seqs, kWaves, kWaves * wave_lds_floats<D, GP>());
  int nwg = 0;
  if (int rc = pkv_split_grid(reinterpret_cast<const void *>(kern), 64 * kWaves, lds, a, &nwg)) return rc;
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(64 * kWaves), lds, reinterpret_cast<hipStream_t>(a.stream), p);
  return (int)hipGetLastError();
}

template <typename E, int D>
int launch_g(const pkv_decode_args &a, const SplitParams &p) {
  if (p.G <= 1) return launch<E, D, 1>(a, p);
  if (p.G <= 2) return launch<E, D, 2>(a, p);
  if (p.G <= 4) return launch<E, D, 4>(a, p);
  if (p.G <= 8) return launch<E, D, 8>(a, p);
  return launch<E, D, 16>(a, p);
}

}  // namespace

int pkv_launch_decode_valu(const pkv_decode_args &a) {
  const SplitParams p = pkv_split_params(a);
  const bool bf = a.L->kv_dtype == PKV_BF16;
  if (a.L->head_dim == 128) return bf ? launch_g<uint16_t, 128>(a, p) : launch_g<float, 128>(a, p);
  return bf ? launch_g<uint16_t, 64>(a, p) : launch_g<float, 64>(a, p);
}
