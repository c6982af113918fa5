// Device-side helpers for the gfx950 kernels: element conversions, DPP
// row reductions, MFMA operand types and the decode kernel parameter block.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_internal.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Unit of token slot t along a row of a one-byte K tile: t with bits 2 and 3
// exchanged.  The score products take a block's slots {0-3, 8-11} into one
// MFMA and {4-7, 12-15} into the other; stored in this order, each of their
// K loads covers whole 128-byte lines instead of halves of twice as many.
__device__ __forceinline__ int k8_unit(int t) { return (t & 3) | ((t & 4) << 1) | ((t & 8) >> 1); }

// Eight bf16 elements of an MFMA operand: a 16-byte unit of a bf16 cache or
// query, or eight one-byte codes (bytes 0..3 of u.x, then of u.y) widened
// exactly to bf16.  An int8 code needs 7 significant bits.  Every FP8 E4M3
// value (3 mantissa bits, exponents -9 .. 8) is a bf16 value too: gfx950's
// scaled conversion, with a scale of 1, widens two codes of one 16-bit half
// straight to bf16 and is exact on all 254 finite codes (checked on the
// device against the format's definition, as the two-step path through a
// float32 pair it replaced), so four instructions widen eight codes.
template <bool F8 = false>
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) {
  return __builtin_bit_cast(bf16x8_t, u);
}
template <bool F8>
__device__ __forceinline__ bf16x8_t as_bf16x8(uint2 u) {
  if constexpr (F8) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.x, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.x, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.y, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.y, 1.0f, true);
    return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else {
    bf16x8_t r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      r[k] = (__bf16)(float)(int8_t)(u.x >> (8 * k));
      r[4 + k] = (__bf16)(float)(int8_t)(u.y >> (8 * k));
    }
    return r;
  }
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
// Zero the one-byte codes of u (bytes 0..3 of u.x, then of u.y) whose index
// is >= nvalid (0..8).  Code 0 is +0 in int8 and in FP8 E4M3.
__device__ __forceinline__ uint2 keep_first(uint2 u, int nvalid) {
  const uint32_t mx = nvalid >= 4 ? 0xffffffffu : (1u << (8 * nvalid)) - 1u;
  const uint32_t my = nvalid >= 8 ? 0xffffffffu : nvalid <= 4 ? 0u : (1u << (8 * (nvalid - 4))) - 1u;
  return make_uint2(u.x & mx, u.y & my);
}

// Loads of cache tiles.  With NT the load carries the non-temporal hint
// (global_load ... nt): the line is streamed through the caches instead of
// being kept for reuse.  A batch that reads each K/V tile once streams HBM
// faster that way (a probe of random 4 KiB tiles: about 6.5 TB/s against
// 5.9 TB/s with cached loads); tiles shared by many sequences are better
// left cached.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <bool NT>
__device__ __forceinline__ uint4 load_u4(const void *p) {
  if constexpr (NT) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const uint4 *>(p);
  }
}
template <bool NT>
__device__ __forceinline__ uint2 load_u2(const void *p) {
  if constexpr (NT) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
    return make_uint2(v.x, v.y);
  } else {
    return *reinterpret_cast<const uint2 *>(p);
  }
}
template <bool NT>
__device__ __forceinline__ float4 load_f4(const void *p) {
  const uint4 u = load_u4<NT>(p);
  return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Clamp a sequence length into what its table can address and what the
// launch grid covers.
__device__ __forceinline__ int clamp_len(int n, int max_blocks, int max_ctx) {
  n = n < 0 ? 0 : n;
  const int cap = max_blocks * 16 < max_ctx ? max_blocks * 16 : max_ctx;
  return n > cap ? cap : n;
}

// Clamp a physical block id into the pool so a corrupt table cannot address
// memory outside it.
__device__ __forceinline__ int clamp_block(int b, int num_blocks) {
  b = b < 0 ? 0 : b;
  return b >= num_blocks ? num_blocks - 1 : b;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// DPP controls: quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
#define PKV_DPP_XOR1 0xB1
#define PKV_DPP_XOR2 0x4E
#define PKV_DPP_HALF_MIRROR 0x141
#define PKV_DPP_MIRROR 0x140

// All-reduce within each 16-lane row.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<PKV_DPP_XOR1>(x));
  x = fmaxf(x, dpp<PKV_DPP_XOR2>(x));
  x = fmaxf(x, dpp<PKV_DPP_HALF_MIRROR>(x));
  x = fmaxf(x, dpp<PKV_DPP_MIRROR>(x));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<PKV_DPP_XOR1>(x);
  x += dpp<PKV_DPP_XOR2>(x);
  x += dpp<PKV_DPP_HALF_MIRROR>(x);
  x += dpp<PKV_DPP_MIRROR>(x);
  return x;
}
// Reduce across the four rows of a wave (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float rows_sum4(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}
__device__ __forceinline__ float rows_max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

// The same across the four rows with the gfx950 lane swaps: the 32-lane swap
// pairs lane l with l ^ 32, the 16-lane swap row r with row r ^ 1; no LDS.
__device__ __forceinline__ float rows_max4_swap(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Balanced split of a decode batch over persistent waves.
//
// The work of a decode step is the list of 32-token chunks of every
// (kv head g, sequence b) segment, ordered by g, then b, then chunk.  Each
// wave of the grid takes one contiguous, equal share of that list (+-1
// chunk), so every wave streams the same number of K/V bytes whatever the
// mix of context lengths, and all waves finish together.  Head-major order
// puts each XCD (one contiguous eighth of the shares, xcd_logical) on about
// one kv head, so blocks read by many sequences -- a shared prompt -- are
// served from that XCD's L2 after their first read.  A segment held by one
// wave is normalised and written out directly.  A segment cut by share
// boundaries leaves one partial result (m, l, o) per wave that touched it, in
// that wave's slot for its first or its last segment (a share is contiguous,
// so only those two can be cut); the merge kernel combines them.

// Parameters of the balanced decode kernels (passed by value).
struct SplitParams {
  float *out;             // [B][Hq][D]
  const void *q;          // [B][Hq][D]
  const void *k_pool;
  const void *v_pool;
  const int32_t *tables;  // [B][max_blocks]
  const int32_t *ctx;     // [B]
  float *ws_o;            // [nslots][G][D] partial outputs
  float *ws_ml;           // [nslots][G][2] partial (max, sum)
  int32_t *ws_hdr;        // [PKV_HDR_INTS + B]: chunks per kv head, waves used, regions,
                          // region bounds (int64), inclusive chunk scan
  int32_t B;
  int32_t num_blocks;
  int32_t H;
  int32_t Hq;
  int32_t G;
  int32_t max_blocks;
  int32_t max_ctx;
  int32_t nslots;         // partial slots, two per wave (bounds every slot index)
  int32_t min_cpw;        // fewest chunks a wave is given
  int32_t ring_off;       // matrix-core kernel: LDS byte offset of wave 0's result ring
  int32_t rec_bytes;      // bytes of one ring record (a piece's G rows, their (m, l), its place)
  int32_t nrec;           // records per wave ring (0: every piece is stored at once)
  int32_t xw[PKV_REGIONS];  // per-XCD weights of the work (all 0: equal shares)
  int32_t *trace;         // nullable: per wave, its XCD group, chunks and start/end times
  float scale_log2;
  int32_t wg_dealt;       // 1: shares follow the workgroups as dealt to the XCDs (round robin)
  int32_t *plan;          // nullable: [B] clamped lengths (padded to 4), then plan_cap records
                          // of PKV_PLAN_REC_INTS (a wave's share and first chunks)
  int32_t plan_cap;       // records the plan holds (every wave that can receive work)
};

// Parameters of the paged prefill kernel (passed by value).
struct PrefillParams {
  float *out;             // [T][Hq][D]
  const void *q;          // [T][Hq][D] bf16
  const void *k_pool;
  const void *v_pool;
  const int32_t *tables;  // [B][max_blocks]
  const int32_t *ctx;     // [B] tokens held, the new ones included
  const int32_t *qstart;  // [B + 1] first query row of each sequence
  int32_t B;
  int32_t num_blocks;
  int32_t H;
  int32_t Hq;
  int32_t G;
  int32_t max_blocks;
  int32_t max_ctx;
  float scale_log2;
};

// Scalar (uniform) load of a read-only int32 through the constant address
// space, so block ids and lengths live in SGPRs and never wait behind the
// vector K/V loads.
typedef const int32_t __attribute__((address_space(4))) *pkv_const_i32;
__device__ __forceinline__ int sload_i32(const int32_t *p) { return *(pkv_const_i32)p; }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Chunks of a sequence of (clamped) length n.
__device__ __forceinline__ int chunks_of(int n) { return (n + 31) >> 5; }

// Inclusive scan of chunk counts over the batch into s_incl[0..B) and the
// clamped lengths into s_len[0..B) (LDS), by all 64*W threads of the
// workgroup.  Returns the total (chunks per kv head).
template <int W>
__device__ int scan_chunks(const SplitParams &P, int32_t *s_incl, int32_t *s_len, int32_t *s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int NT = 64 * W;
  const int per = (P.B + NT - 1) / NT;
  const int i0 = tid * per, i1 = min(i0 + per, P.B);
  int local = 0;
  for (int i = i0; i < i1; ++i) {
    const int n = clamp_len(P.ctx[i], P.max_blocks, P.max_ctx);
    const int c = chunks_of(n);
    s_len[i] = n;
    s_incl[i] = c;
    local += c;
  }
  int v = local;  // inclusive scan across the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  if (lane == 63) s_wave[w] = v;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int k = 0; k < W; ++k) {
    const int t = s_wave[k];
    base += k < w ? t : 0;
    total += t;
  }
  int run = base + v - local;
  for (int i = i0; i < i1; ++i) {
    run += s_incl[i];
    s_incl[i] = run;
  }
  __syncthreads();
  return total;
}

// Waves that receive work: all of them, unless that would give a wave fewer
// than min_cpw chunks.
__device__ __forceinline__ int waves_used(int64_t c_tot, int nw, int min_cpw) {
  const int64_t cap = c_tot / min_cpw;
  return (int)max((int64_t)1, min((int64_t)nw, cap));
}

// Regions of the chunk list.  With per-XCD weights the list is cut into 8
// regions, region r sized by weight r and shared equally by the waves of
// XCD r; otherwise one region holds the whole list.  bounds[0..nr] are the
// region starts (int64, in LDS or in the schedule header), so that
// wave_of, and the share of every wave, follow from them exactly alike in
// the decode and merge kernels.
struct Regions {
  int64_t C;
  int nwe, nr, wpr;
  const int64_t *bounds;  // nr + 1 entries

  // Region holding chunk x.
  __device__ int region_of(int64_t x) const {
    int r = 0;
    for (int i = 1; i < nr; ++i) r = x >= bounds[i] ? i : r;
    return r;
  }
  // Wave whose share holds chunk x (shares are [R + i*S/wpr, R + (i+1)*S/wpr)
  // within region r = [R, R + S)).
  __device__ int wave_of(int64_t x) const {
    const int r = region_of(x);
    const int64_t R = bounds[r], S = bounds[r + 1] - R;
    return r * wpr + (int)(((x - R + 1) * wpr - 1) / S);
  }
  __device__ void share(int w, int64_t &lo, int64_t &hi) const {
    const int r = w / wpr, i = w - r * wpr;
    const int64_t R = bounds[r], S = bounds[r + 1] - R;
    lo = R + (int64_t)i * S / wpr;
    hi = R + (int64_t)(i + 1) * S / wpr;
  }
};

// Region bounds of a launch into b[0..PKV_REGIONS]; returns the region
// count.  Weights apply when every XCD holds the same number of used waves
// (the whole grid works, and workgroups spread evenly over the 8 XCDs),
// every weight is positive, and every wave's share keeps min_cpw chunks;
// otherwise there is one region.
__device__ inline int region_bounds(int64_t c_tot, int nwe, int nwg_waves, int nwg, const int32_t *xw,
                                    int min_cpw, int64_t *b) {
  int64_t wsum = 0;
  bool pos = true;
#pragma unroll
  for (int i = 0; i < PKV_REGIONS; ++i) {
    wsum += xw[i];
    pos = pos && xw[i] > 0;
  }
  b[0] = 0;
  // c_tot * (a partial weight sum) must fit in int64 for the bounds to be
  // exact and increasing.
  if (pos && nwe == nwg_waves && nwg % PKV_REGIONS == 0 && wsum < (1 << 24) &&
      c_tot < ((int64_t)1 << 62) / wsum) {
    const int wpr = nwe / PKV_REGIONS;
    int64_t cum = 0;
    bool ok = true;
#pragma unroll
    for (int i = 0; i < PKV_REGIONS; ++i) {
      cum += xw[i];
      b[i + 1] = i + 1 == PKV_REGIONS ? c_tot : c_tot * cum / wsum;
      ok = ok && (b[i + 1] - b[i]) / wpr >= min_cpw;
    }
    if (ok) return PKV_REGIONS;
  }
  b[1] = c_tot;
  return 1;
}

// Workgroups are dealt round-robin to the 8 XCDs; renumber them so that each
// XCD holds one contiguous eighth of the shares (neighbouring shares often
// read the same segment's query and table lines, which then stay in one L2,
// and a kv head's blocks shared by many sequences are read by one XCD).
// One-byte caches without sharing keep the dealt order (see the launcher).
__device__ __forceinline__ int xcd_logical(int wg, int nwg) {
  return (nwg & 7) ? wg : (wg & 7) * (nwg >> 3) + (wg >> 3);
}

// LDS of a decode workgroup: the chunk scan, the clamped lengths and W wave
// totals, padded to 16 bytes (int32 units: pkv_split_lds_ints), then
// extra_floats of per-wave slices.
__host__ __device__ inline int pkv_split_lds_ints(int num_seqs, int waves) {
  return ((2 * num_seqs + waves + 3) & ~3) + 2 * (PKV_REGIONS + 1) + 2;
}
// Offset (int32 units) of the region bounds in a decode workgroup's LDS.
__host__ __device__ inline int pkv_split_bounds_ints(int num_seqs, int waves) { return (2 * num_seqs + waves + 3) & ~3; }
inline size_t pkv_split_lds_bytes(int num_seqs, int waves, int extra_floats = 0) {
  return (size_t)pkv_split_lds_ints(num_seqs, waves) * sizeof(int32_t) + (size_t)extra_floats * sizeof(float);
}

inline SplitParams pkv_split_params(const pkv_decode_args &a) {
  SplitParams p;
  p.out = a.out;
  p.q = a.q;
  p.k_pool = a.k_pool;
  p.v_pool = a.v_pool;
  p.tables = a.tables;
  p.ctx = a.ctx;
  p.ws_o = a.ws_o;
  p.ws_ml = a.ws_ml;
  p.ws_hdr = a.ws_hdr;
  p.B = a.num_seqs;
  p.num_blocks = a.L->num_blocks;
  p.H = a.L->num_kv_heads;
  p.Hq = a.num_q_heads;
  p.G = a.num_q_heads / a.L->num_kv_heads;
  p.max_blocks = a.max_blocks;
  p.max_ctx = a.max_ctx;
  p.nslots = a.nslots;
  p.min_cpw = a.min_cpw;
  p.ring_off = 0;
  p.rec_bytes = 0;
  p.nrec = 0;
  for (int i = 0; i < PKV_REGIONS; ++i) p.xw[i] = a.xw[i];
  p.trace = a.trace;
  p.scale_log2 = a.scale_log2;
  p.wg_dealt = 0;
  p.plan = a.plan_mode ? a.plan : nullptr;
  p.plan_cap = a.plan_mode ? a.plan_cap : 0;
  return p;
}

// Position of a wave in the chunk list: sequence b, kv head g, chunk j of the
// segment, the segment's chunk count and length, and the list index of the
// segment's first chunk.  All wave-uniform (SGPRs).
struct Cursor {
  int b, g, j, cnt, n;
  int64_t seg0;
};

// One wave's share [lo, hi) of the chunk list and the walk through it.  The
// chunk scan and the clamped lengths are in LDS (GL false: the kernel's own
// scan) or in device memory (GL true: a plan's), read with scalar loads.
template <bool GL>
struct ShareT {
  const int32_t *s_incl;  // inclusive chunk scan over the batch
  const int32_t *s_len;   // clamped lengths
  const int32_t *ctx;
  const int32_t *tables;
  int B, max_blocks, max_ctx, num_blocks;
  int64_t c_seq, c_tot;
  int nwe, wave;
  int64_t lo, hi;
  Regions rg;

  __device__ int at(const int32_t *p, int i) const {
    if constexpr (GL)
      return sload_i32(p + i);
    else
      return uniform(p[i]);
  }
  __device__ int cnt_of(int b) const { return at(s_incl, b) - (b ? at(s_incl, b - 1) : 0); }
  __device__ int len_of(int b) const { return at(s_len, b); }

  // The share's first chunk: kv head lo / c_seq, then the first sequence
  // whose chunks end past the remainder.
  __device__ Cursor first() const {
    Cursor c;
    c.g = (int)(lo / c_seq);
    const int rem = (int)(lo - (int64_t)c.g * c_seq);
    int a = 0, z = B - 1;
    while (a < z) {
      const int mid = (a + z) >> 1;
      if (at(s_incl, mid) > rem)
        z = mid;
      else
        a = mid + 1;
    }
    c.b = a;
    c.cnt = cnt_of(a);
    const int excl = at(s_incl, a) - c.cnt;
    c.j = rem - excl;
    c.n = len_of(a);
    c.seg0 = (int64_t)c.g * c_seq + excl;
    return c;
  }

  // The next chunk in list order (call only while one remains in the share).
  // Segments are contiguous in the list, so the next one starts where this
  // one ends; empty sequences are skipped.
  __device__ Cursor next(Cursor c) const {
    if (++c.j < c.cnt) return c;
    c.j = 0;
    c.seg0 += c.cnt;
    do {
      if (++c.b == B) {
        c.b = 0;
        ++c.g;
      }
    } while (cnt_of(c.b) == 0);
    c.cnt = cnt_of(c.b);
    c.n = len_of(c.b);
    return c;
  }

  // Physical blocks of a chunk; the second is the first again when the chunk
  // holds no token of it (only the last chunk of a segment can).
  // Both entries are read at once (the second at a row-clamped index, so it
  // never waits for the length and never leaves the row).
  __device__ void blocks(const Cursor &c, int &pa, int &pb) const {
    const int32_t *row = tables + (size_t)c.b * max_blocks;
    const int a = sload_i32(row + 2 * c.j);
    const int b2 = sload_i32(row + min(2 * c.j + 1, max_blocks - 1));
    pa = clamp_block(a, num_blocks);
    pb = (32 * c.j + 16 < c.n) ? clamp_block(b2, num_blocks) : pa;
  }

  // Whether this wave holds every chunk of the cursor's segment.
  __device__ bool whole(const Cursor &c) const { return c.seg0 >= lo && c.seg0 + c.cnt <= hi; }

  // Partial slot of this wave for a cut segment: 2 wave when it is the
  // wave's first segment (its share starts inside it), 2 wave + 1 when it is
  // its last (< nslots by construction; clamped so that a broken invariant
  // cannot write outside the workspace).
  __device__ int slot(const Cursor &c, int nslots) const { return min(2 * wave + (lo < c.seg0 ? 1 : 0), nslots - 1); }
};
using Share = ShareT<false>;

// Plan record of one wave (PKV_PLAN_REC_INTS int32): lo and hi of its share
// (int64 each), then for each of its first PKV_PLAN_CHUNKS chunks, 16-byte
// aligned, the cursor (b, g, j, cnt, n, seg0 as two ints) and the two
// physical blocks.
constexpr int kPlanCursorInts = 12;
static_assert(4 + kPlanCursorInts * PKV_PLAN_CHUNKS <= PKV_PLAN_REC_INTS, "a plan record holds its chunks");

// Common start of the balanced-split kernels: the chunk scan (all threads),
// the merge kernel's schedule header and zero rows for empty sequences
// (workgroup 0), and this wave's share.  Returns false when the wave has no
// work.
template <int W, int D>
__device__ bool split_begin(const SplitParams &P, int32_t *s_lds, Share &sh) {
  const int tid = threadIdx.x, w = tid >> 6;
  int32_t *s_incl = s_lds, *s_len = s_lds + P.B, *s_wave = s_lds + 2 * P.B;
  const int64_t c_seq = scan_chunks<W>(P, s_incl, s_len, s_wave);
  const int64_t c_tot = (int64_t)P.H * c_seq;
  const int nwg = gridDim.x;
  const int nwe = waves_used(c_tot, nwg * W, P.min_cpw);
  int64_t *s_bounds = reinterpret_cast<int64_t *>(s_lds + pkv_split_bounds_ints(P.B, W));
  int32_t *s_nr = s_lds + pkv_split_bounds_ints(P.B, W) + 2 * (PKV_REGIONS + 1);
  if (tid == 0) *s_nr = region_bounds(c_tot, nwe, nwg * W, nwg, P.xw, P.min_cpw, s_bounds);
  __syncthreads();
  const int nr = *s_nr;
  if (blockIdx.x == 0) {
    if (tid == 0) {
      P.ws_hdr[0] = (int32_t)c_seq;
      P.ws_hdr[1] = nwe;
      P.ws_hdr[2] = nr;
      P.ws_hdr[3] = 0;
    }
    if (tid <= nr) reinterpret_cast<int64_t *>(P.ws_hdr + 4)[tid] = s_bounds[tid];
    // Each thread takes its own sequences, so this workgroup starts
    // streaming as early as the others (a walk over the whole batch by
    // every thread cost it microseconds); an empty sequence (padding) has
    // its rows zeroed by the thread that found it.
    for (int b = tid; b < P.B; b += 64 * W) {
      P.ws_hdr[PKV_HDR_INTS + b] = s_incl[b];
      if (P.plan) P.plan[b] = s_len[b];  // a plan's walk reads the lengths from memory
      if (P.out && s_incl[b] == (b ? s_incl[b - 1] : 0)) {  // no output when planning
        float *row = P.out + (size_t)b * P.Hq * D;  // out is only 4-byte aligned
        for (int i = 0; i < P.Hq * D; ++i) row[i] = 0.f;
      }
    }
  }
  sh.s_incl = s_incl;
  sh.s_len = s_len;
  sh.ctx = P.ctx;
  sh.tables = P.tables;
  sh.B = P.B;
  sh.max_blocks = P.max_blocks;
  sh.max_ctx = P.max_ctx;
  sh.num_blocks = P.num_blocks;
  sh.c_seq = c_seq;
  sh.c_tot = c_tot;
  sh.nwe = nwe;
  sh.rg.C = c_tot;
  sh.rg.nwe = nwe;
  sh.rg.nr = nr;
  sh.rg.wpr = nwe / nr;
  sh.rg.bounds = s_bounds;
  sh.wave = uniform((P.wg_dealt ? (int)blockIdx.x : xcd_logical(blockIdx.x, nwg)) * W + w);
  if (sh.wave >= nwe || c_tot == 0) return false;
  sh.rg.share(sh.wave, sh.lo, sh.hi);
  return sh.lo < sh.hi;
}
