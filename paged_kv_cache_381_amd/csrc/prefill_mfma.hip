// Paged prefill: causal attention of a sequence's new tokens over its paged
// cache, on the matrix cores (bf16, int8 or FP8 cache).
//
// What it computes [KV Cache 工程学 §15.1: a prompt is a causal i x i
// attention; §15.6 and 新一代 KV Cache 管理 §8.3: a cached prefix is not
// prefilled again]: sequence b holds ctx_b tokens in its table, the last
// nq_b of them new (their K/V already stored by paged_kv_append).  New token t
// sits at position p_b + t, p_b = ctx_b - nq_b, and attends to positions
// 0 .. p_b + t -- the cached prefix and the new tokens up to itself.
//
// gfx950 mapping.  The decode kernel's contractions are reused with the
// padding gone: a column tile is 16 query columns, TQ = 16 / G consecutive
// new tokens times the G query heads of one kv head g, so every column of
//   S^T[32 keys x 16 columns] = K[32 x D] . Q^T[D x 16]
//   O^T[D x 16 columns]      += V^T[D x 32] . P^T[32 x 16]
// is a real query row.  The operand layouts, the lane holding 8 keys of one
// column between the two products and the online softmax per column are the
// decode kernel's; the causal limit differs per column and masks scores per
// lane.  A wave takes CT column tiles (the K and V operands of each chunk
// serve all of them) and walks keys 0 .. its last token's position in
// 32-key chunks (two blocks through the table), with a ring of NB chunks of
// K/V in registers, every load issued on every path so that the
// memory-counter waits stay exact; the query slices wait in LDS.  Two waves
// share each SIMD.  Tiles that run longest (the last tokens) are dispatched
// first, across all (sequence, kv head) pairs.
//
// Per chunk the wave forms the next chunk's scores while it weighs this
// one's, so the matrix products and the exponentials of one step are
// independent.  Weights are checked after the fact: a weight above 2^8 (an
// overflow against a stale running maximum) sends the wave down a rare path
// that moves the maximum, rescales and weighs again; bf16 weights are
// non-negative, so the check is an integer maximum of their bit patterns.
// Chunks below every column's causal limit skip masking entirely.  bf16 row
// sums come from the matrix cores (a ones operand against the rounded
// weights).
#include <algorithm>
#include <type_traits>
#include <utility>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace {

constexpr float kSlack = 8.0f;  // headroom of the running maximum (base 2)

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Eight floats rounded to bf16 (nearest even), two per conversion.
__device__ __forceinline__ bf16x8_t pack_bf16x8(const float (&e)[8]) {
  uint4 u;
  u.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{e[0], e[1]}, bf16x2_t));
  u.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{e[2], e[3]}, bf16x2_t));
  u.z = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{e[4], e[5]}, bf16x2_t));
  u.w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{e[6], e[7]}, bf16x2_t));
  return __builtin_bit_cast(bf16x8_t, u);
}

template <int D, int NB, bool I8, int CT, bool F8>
// Two waves per SIMD (at most 256 registers a wave): one wave alone issues
// its matrix products at about 60 % of the matrix cores' rate and cannot run
// them beside its own vector work, two keep the matrix cores busier while
// the other wave weighs.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_mfma_kernel(
    PrefillParams P) {
  constexpr int NKK = D / 32;
  constexpr int NNN = D / 16;
  constexpr int TB = I8 ? 16 * D + 64 : 32 * D;
  constexpr int NKU = I8 ? NKK / 2 : NKK;
  using VUnit = std::conditional_t<I8, uint2, uint4>;
  // One-byte caches: each of the two waves on a SIMD raises its priority
  // over its matrix products, so the SIMD issues one wave's products while
  // the other wave's widening and weighing fill the gaps (measured +5 %);
  // the bf16 kernel, with less vector work per chunk, loses 5 % with it.
  constexpr bool PRIO = I8;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: the walk's bounds live in SGPRs
  // Workgroup x takes the (x / (H B))-th group of four waves, counted from
  // the last new tokens, of kv head x % H of sequence (x / H) % B: workgroups
  // are dispatched in order, so the longest walks of every (sequence, kv
  // head) start first and the short ones fill the end, instead of one
  // sequence's and head's long walks starting last and running alone.
  // Consecutive workgroups go to the XCDs in turn, so with H B a multiple of
  // 8 each XCD keeps to the kv heads g = x % 8 and its L2 to their blocks.
  const int g = (int)(blockIdx.x % P.H);
  const int b = (int)((blockIdx.x / P.H) % P.B);
  const int wg = (int)(blockIdx.x / ((unsigned)P.H * P.B));
  const int G = P.G, TQ = 16 / G;
  const int q0 = sload_i32(P.qstart + b);
  const int n = clamp_len(sload_i32(P.ctx + b), P.max_blocks, P.max_ctx);
  // A sequence claiming more new tokens than it holds keeps its last n.
  const int nq = min(sload_i32(P.qstart + b + 1) - q0, n);
  const int ntile = (nq + TQ - 1) / TQ;
  // The wave's CT column tiles, longest first; tiles run longest first too.
  const int t_first = ntile - 1 - (wg * 4 + w) * CT;
  if (t_first < 0) return;
  const int p0 = n - nq;  // position of new token 0
  const int kend = p0 + min(t_first * TQ + TQ, nq);  // keys the wave's last token sees
  const int nch = (kend + 31) >> 5;

  // Scores stay unscaled (the scale joins the exponent's fma) unless the
  // scale is not positive or int8 keys carry their own scales.
  const bool raw = !I8 && P.scale_log2 > 0.f;
  const float mul = raw ? P.scale_log2 : 1.f;
  // The earliest column's causal limit: chunks up to it are open to all
  // columns and need no mask.  The open walk ends on a ring boundary.
  const int pos_min = p0 + max(t_first - CT + 1, 0) * TQ;
  const int c_open = raw ? min((pos_min + 1) >> 5, nch) / NB * NB : 0;

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

  // The query slices stay in LDS for the whole walk, each lane's own 16
  // bytes per (tile, score step), and are read again at each use (a volatile
  // LDS read, so the compiler does not hoist them into registers: the
  // registers go to the K/V ring and the accumulators).
  __shared__ uint4 s_q[4][CT][NKK][64];
#pragma unroll
  for (int s = 0; s < CT; ++s) {
    const uint4 *qr = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(P.q) + qrow[s] * D);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) s_q[w][s][kk][lane] = qr[kgroup(kk)];
  }
  auto qslice = [&](int s, int kk) {
    typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
    typedef const volatile __attribute__((address_space(3))) u32x4v lds_u32x4v;
    const u32x4v v = *(lds_u32x4v *)(&s_q[w][s][kk][lane]);
    return __builtin_bit_cast(bf16x8_t, v);
  };

  // Chunk y lives in ring slot y % NB of the K ring and of the V ring.  Its
  // K is requested NB steps before its scores are formed (one step before
  // its weights are applied), its V -- with the int8 scales of K and V -- NB
  // steps before the V product.  Chunks past the walk's end re-read its
  // last chunk: every load is issued on every path, and what they bring is
  // masked.
  int ka[NB], kb[NB], va_blk[NB], vb_blk[NB];
  uint4 ax[NB][NKU], ay[NB][NKU];
  VUnit va[NB][NNN];
  float4 ksc[NB][2], vsc[NB][2];

  auto locate = [&](int &pa, int &pb, int y) {
    const int c = min(y, nch - 1);
    pa = clamp_block(sload_i32(trow + 2 * c), P.num_blocks);
    const int b2 = clamp_block(sload_i32(trow + min(2 * c + 1, P.max_blocks - 1)), P.num_blocks);
    pb = 32 * c + 16 < kend ? b2 : pa;
  };
  auto issue_k = [&](auto bi, int y) {
    constexpr int I = decltype(bi)::value;
    locate(ka[I], kb[I], y);
    const uint4 *kt = reinterpret_cast<const uint4 *>(kpool + ((size_t)(ksel ? kb[I] : ka[I]) * H + g) * TB);
#pragma unroll
    for (int ku = 0; ku < NKU; ++ku) {
      const int cu = 4 * ku + grp;
      ax[I][ku] = kt[cu * 16 + (I8 ? k8_unit(ktx) : ktx)];
      ay[I][ku] = kt[cu * 16 + (I8 ? k8_unit(ktx + 4) : ktx + 4)];
    }
  };
  auto issue_v = [&](auto bi, int y) {
    constexpr int I = decltype(bi)::value;
    locate(va_blk[I], vb_blk[I], y);
    const size_t tile = ((size_t)(vsel ? vb_blk[I] : va_blk[I]) * H + g) * TB;
    const uint8_t *vt = vpool + tile;
    if constexpr (I8) {
#pragma unroll
      for (int nn = 0; nn < NNN; ++nn) va[I][nn] = *reinterpret_cast<const uint2 *>(vt + (16 * nn + r16) * 16 + 8 * vhalf);
      const float4 *kq = reinterpret_cast<const float4 *>(kpool + tile + 16 * D + 32 * vhalf);
      const float4 *vq = reinterpret_cast<const float4 *>(vt + 16 * D + 32 * vhalf);
      ksc[I][0] = kq[0];
      ksc[I][1] = kq[1];
      vsc[I][0] = vq[0];
      vsc[I][1] = vq[1];
    } else {
      const uint4 *u = reinterpret_cast<const uint4 *>(vt);
#pragma unroll
      for (int nn = 0; nn < NNN; ++nn) va[I][nn] = u[2 * (16 * nn + r16) + vhalf];
    }
  };
  // Scores of the chunk whose K sits in slot I: 32 keys x 16 columns.
  auto scores = [&](auto bi, f32x4_t (&sx)[CT], f32x4_t (&sy)[CT]) {
    constexpr int I = decltype(bi)::value;
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < CT; ++s) sx[s] = sy[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bf16x8_t kx, ky;
      if constexpr (I8) {
        const uint4 ux = ax[I][kk >> 1], uy = ay[I][kk >> 1];
        kx = as_bf16x8<F8>((kk & 1) ? make_uint2(ux.z, ux.w) : make_uint2(ux.x, ux.y));
        ky = as_bf16x8<F8>((kk & 1) ? make_uint2(uy.z, uy.w) : make_uint2(uy.x, uy.y));
      } else {
        kx = as_bf16x8<F8>(ax[I][kk]);
        ky = as_bf16x8<F8>(ay[I][kk]);
      }
      bf16x8_t qv[CT];
#pragma unroll
      for (int s = 0; s < CT; ++s) qv[s] = qslice(s, kk);
#pragma unroll
      for (int s = 0; s < CT; ++s) {
        sx[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kx, qv[s], sx[s], 0, 0, 0);
        sy[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ky, qv[s], sy[s], 0, 0, 0);
      }
    }
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
  };

  f32x4_t o[CT][NNN];
  float m[CT];
  // Row sums: bf16 weights are summed on the matrix cores (a ones operand
  // against the same rounded weights the V product uses, so the sum lands
  // in every row of the column); int8 weights carry V's scale, so their
  // plain exponentials are summed per lane.
  f32x4_t lacc[CT];
  float l[CT];
#pragma unroll
  for (int s = 0; s < CT; ++s) {
#pragma unroll
    for (int nn = 0; nn < NNN; ++nn) o[s][nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m[s] = -INFINITY;
    lacc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    l[s] = 0.f;
  }
  bf16x8_t ones;
#pragma unroll
  for (int r = 0; r < 8; ++r) ones[r] = (__bf16)1.0f;

  f32x4_t sx[CT], sy[CT];  // scores of the chunk being weighted
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    ((issue_k(std::integral_constant<int, Is>{}, Is), __builtin_amdgcn_sched_barrier(0),
      issue_v(std::integral_constant<int, Is>{}, Is), __builtin_amdgcn_sched_barrier(0)),
     ...);
  }(std::make_integer_sequence<int, NB>{});
  scores(std::integral_constant<int, 0>{}, sx, sy);
  issue_k(std::integral_constant<int, 0>{}, NB);

  int x = 0;
  // One chunk: weights of chunk x from its scores (sx, sy), the scores of
  // chunk x+1, the V product of chunk x, and the next requests.
  auto step = [&](auto bi, auto open_c) {
    constexpr int I = decltype(bi)::value;
    constexpr int J = (I + 1) % NB;
    constexpr bool OPEN = decltype(open_c)::value;
    const int tb = 32 * x + 16 * vsel + 8 * vhalf;  // this lane's 8 keys: tb .. tb+7
    float ks[8], vs[8];
    if constexpr (I8) {
      ks[0] = ksc[I][0].x; ks[1] = ksc[I][0].y; ks[2] = ksc[I][0].z; ks[3] = ksc[I][0].w;
      ks[4] = ksc[I][1].x; ks[5] = ksc[I][1].y; ks[6] = ksc[I][1].z; ks[7] = ksc[I][1].w;
      vs[0] = vsc[I][0].x; vs[1] = vsc[I][0].y; vs[2] = vsc[I][0].z; vs[3] = vsc[I][0].w;
      vs[4] = vsc[I][1].x; vs[5] = vsc[I][1].y; vs[6] = vsc[I][1].z; vs[7] = vsc[I][1].w;
    }
    int lim[CT];
    if constexpr (!OPEN) {
      // Past each column's causal limit (and past the walk's end) a score
      // is -inf; without the raw form, scores take their scales here.
      const bool real = x < nch;
#pragma unroll
      for (int s = 0; s < CT; ++s) {
        lim[s] = real ? pos[s] : -1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float kx = I8 ? ks[r] : 1.f, ky = I8 ? ks[4 + r] : 1.f;
          const float fx = raw ? 1.f : kx * P.scale_log2, fy = raw ? 1.f : ky * P.scale_log2;
          sx[s][r] = (tb + r <= lim[s]) ? sx[s][r] * fx : -INFINITY;
          sy[s][r] = (tb + 4 + r <= lim[s]) ? sy[s][r] * fy : -INFINITY;
        }
      }
      if constexpr (!I8 || F8) {
        // Keys at or past the walk's end may be unwritten (NaN, also as FP8
        // codes); a zero weight alone would not cancel them.
        const int nvalid = real ? min(max(kend - tb, 0), 8) : 0;
        if (nvalid < 8) {
#pragma unroll
          for (int nn = 0; nn < NNN; ++nn) va[I][nn] = keep_first(va[I][nn], nvalid);
        }
      }
    }

    // Weights against the running maximum; int8 weights take V's scale.
    bf16x8_t pv[CT];
    float psum[CT];
    auto weigh = [&]() {
#pragma unroll
      for (int s = 0; s < CT; ++s) {
        psum[s] = 0.f;
        float e[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float sc = r < 4 ? sx[s][r] : sy[s][r - 4];
          e[r] = fast_exp2(__builtin_fmaf(sc, mul, -m[s]));
          if constexpr (I8) {
            psum[s] += e[r];
            e[r] = (tb + r <= lim[s]) ? e[r] * vs[r] : 0.f;  // scales past the context may be NaN
          }
        }
        pv[s] = pack_bf16x8(e);
      }
    };
    weigh();
    f32x4_t nx[CT], ny[CT];
    scores(std::integral_constant<int, J>{}, nx, ny);
    issue_k(std::integral_constant<int, J>{}, x + 1 + NB);

    // A weight above 2^kSlack (or inf / NaN against the -inf start) means
    // the running maximum must move: rare after the first chunk.  bf16
    // weights are non-negative, so their bit patterns order as integers.
    bool over;
    if constexpr (I8) {
      float emax = 0.f;
#pragma unroll
      for (int s = 0; s < CT; ++s) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float sc = r < 4 ? sx[s][r] : sy[s][r - 4];
          emax = fmaxf(emax, sc * mul - m[s]);
        }
      }
      over = !(emax <= kSlack);
    } else {
      u16x2_t mx = u16x2_t{0, 0};
#pragma unroll
      for (int s = 0; s < CT; ++s) {
        const u16x8_t u = __builtin_bit_cast(u16x8_t, pv[s]);
        mx = __builtin_elementwise_max(mx, __builtin_elementwise_max(__builtin_elementwise_max(u.s01, u.s23),
                                                                      __builtin_elementwise_max(u.s45, u.s67)));
      }
      over = max((unsigned)mx.x, (unsigned)mx.y) > 0x4380u;  // bf16 of 2^kSlack = 256
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(over) != 0, 0)) {
#pragma unroll
      for (int s = 0; s < CT; ++s) {
        float cmax = fmaxf(fmaxf(fmaxf(sx[s][0], sx[s][1]), fmaxf(sx[s][2], sx[s][3])),
                           fmaxf(fmaxf(sy[s][0], sy[s][1]), fmaxf(sy[s][2], sy[s][3])));
        cmax = rows_max4_swap(cmax) * mul;
        const float mnew = fmaxf(m[s], cmax);
        const float alpha = fast_exp2(m[s] - mnew);
        m[s] = mnew;
        l[s] *= alpha;
        lacc[s] *= alpha;
#pragma unroll
        for (int nn = 0; nn < NNN; ++nn) o[s][nn] *= alpha;
      }
      weigh();
    }

    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < CT; ++s) {
      if constexpr (I8)
        l[s] += psum[s];
      else
        lacc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pv[s], lacc[s], 0, 0, 0);
    }
#pragma unroll
    for (int nn = 0; nn < NNN; ++nn) {
      const bf16x8_t vop = as_bf16x8<F8>(va[I][nn]);
#pragma unroll
      for (int s = 0; s < CT; ++s) o[s][nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pv[s], o[s][nn], 0, 0, 0);
    }
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    issue_v(std::integral_constant<int, I>{}, x + NB);
#pragma unroll
    for (int s = 0; s < CT; ++s) {
      sx[s] = nx[s];
      sy[s] = ny[s];
    }
    ++x;
  };
  while (x < c_open) {
    [&]<int... Is>(std::integer_sequence<int, Is...>) {
      (step(std::integral_constant<int, Is>{}, std::true_type{}), ...);
    }(std::make_integer_sequence<int, NB>{});
  }
  while (x < nch) {
    [&]<int... Is>(std::integer_sequence<int, Is...>) {
      (step(std::integral_constant<int, Is>{}, std::false_type{}), ...);
    }(std::make_integer_sequence<int, NB>{});
  }

#pragma unroll
  for (int s = 0; s < CT; ++s) {
    const float lsum = I8 ? rows_sum4(l[s]) : lacc[s][0];
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

// Ring depth (chunks of K/V requested ahead) and column tiles per wave (16
// query columns each: the K and V operands of a chunk serve all of them, so
// each byte brought through the vector memory path feeds CT x the math).
// Three tiles and one ring slot fit two waves per SIMD in 256 registers
// each, with the query slices in LDS (bf16 and one-byte caches alike; two
// ring slots spill).  A wave's next chunk is then requested one step ahead,
// and the other wave on the SIMD covers the wait.
#ifndef PKV_PREFILL_NBUF
#define PKV_PREFILL_NBUF 1
#endif
#ifndef PKV_PREFILL_CT
#define PKV_PREFILL_CT 3
#endif
#ifndef PKV_PREFILL_NBUF_I8
#define PKV_PREFILL_NBUF_I8 1
#endif
#ifndef PKV_PREFILL_CT_I8
#define PKV_PREFILL_CT_I8 3
#endif

// I8: one-byte codes (int8, or FP8 E4M3 when F8) with per-row scales.
template <int D, bool I8, bool F8 = false>
int launch(const pkv_prefill_args &a, const PrefillParams &p) {
  constexpr int CT = I8 ? PKV_PREFILL_CT_I8 : PKV_PREFILL_CT;
  auto kern = prefill_mfma_kernel<D, I8 ? PKV_PREFILL_NBUF_I8 : PKV_PREFILL_NBUF, I8, CT, F8>;
  const int tq = 16 / p.G;
  const int tiles = (a.max_query_len + tq - 1) / tq;
  const int waves = (tiles + CT - 1) / CT;
  const int64_t nwg = (int64_t)((waves + 3) / 4) * p.H * a.num_seqs;
  if (nwg > 0x7fffffff) return (int)hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(256), 0, reinterpret_cast<hipStream_t>(a.stream), p);
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
  p.B = a.num_seqs;
  if (a.L->kv_dtype == PKV_INT8) return a.L->head_dim == 128 ? launch<128, true>(a, p) : launch<64, true>(a, p);
  if (a.L->kv_dtype == PKV_FP8)
    return a.L->head_dim == 128 ? launch<128, true, true>(a, p) : launch<64, true, true>(a, p);
  return a.L->head_dim == 128 ? launch<128, false>(a, p) : launch<64, false>(a, p);
}
