// PagedAttention decode, matrix-core kernel (bf16 or int8 KV, grouped-query
// heads).
//
// What it computes [KV Cache 工程学 §15.5; 新一代 KV Cache 管理 §8.1]: for a
// sequence b and its query heads h of kv group g, the new token's query is
// dotted with the K of every cached token, found by reading block-table entry
// j/16 and slot j%16; a softmax over the whole context weights the cached V.
// The context is visited 32 tokens at a time with a running maximum and sum
// (online softmax), so the softmax stays global even though the data arrive
// block by block (the per-page softmax of the vendor article
// [PagedAttention：大模型KV Cache内存管理革新 §3.2] is not used).  The
// maximum used as the exponent's reference only moves when new scores exceed
// it by more than 2^8 in weight; any reference gives the same quotient, and
// skipping the rescale of the D/16 accumulator tiles saves most of the
// per-chunk vector work.
//
// Work split.  Persistent waves each take one equal, contiguous share of the
// batch's 32-token chunks (pkv_device.h, "Balanced split"): the mix of
// context lengths does not leave a tail of long sequences running alone.
// Within its share a wave walks (sequence, kv head) segments in order; a
// segment it holds entirely is normalised and stored, a segment cut by a share
// boundary leaves a partial (m, l, o) in the wave's slot for the merge
// kernel.
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
// xor-shuffles per chunk (max over the four lane groups).  The first MFMA's
// K rows are thus slots {0-3, 8-11} of each block and the second's {4-7,
// 12-15}: a bf16 K load reads half of each 128-byte line it touches, while
// one-byte K tiles store the slots in that order (k8_unit), so each of their
// K loads reads whole lines, which matters once the loads stream.  Each lane
// holds the 8-element slices of the group's query rows that its B operand
// needs (D/32 16-byte loads per lane), one set per pipeline buffer, loaded
// when a buffer moves to a chunk of another segment and kept while the
// segment lasts; the whole group shares them through the MFMA, and nothing
// else in the wave would reuse an LDS copy.
//
// int8 cache [KV Cache 工程学 §15.7 (3)].  Codes are loaded 8 bytes per lane
// where bf16 takes 16 and widened to bf16 exactly (|code| <= 127 needs 7
// significant bits), so the same MFMAs run on the same lane layout.  A
// token's K scale multiplies its score after the score MFMA; its V scale
// multiplies its softmax weight before the weight is rounded to bf16 for the
// PV MFMA, while the running sum takes the weight itself.  Each lane reads the
// 8 scales of its 8 token slots (32 contiguous bytes) of K and of V.  Int8
// codes of slots past the context are finite whatever they hold, so a zero
// weight masks them; their scales may be anything and are never used.
//
// FP8 E4M3 cache: the same tiles, scales and lane layout; the gfx950
// conversion instruction widens two codes at a time, exactly, to bf16.  Two
// of its codes are NaN, so V codes past the context are zeroed as bf16
// elements are.
//
// Memory pipeline.  NB register buffers of K/V (two by default): the step
// that computes chunk c requests chunk c+NB-1 into the buffer chunk c-1
// used, its K right after chunk c's score MFMAs and its V right after the PV
// MFMAs, then locates chunk c+NB (block ids: scalar loads) into the buffer it
// has just consumed and, when that chunk opens another segment, requests its
// query slices; so a wave always has loads in flight through its own math.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace {

// s_waitcnt immediate of gfx9 waiting for no outstanding vector memory
// operation (vmcnt 0) and leaving the other counters unchecked.
constexpr int kDrainVm = 0x0F70;

// Headroom of the running maximum, in base-2 exponent units: a chunk whose
// scores stay within 2^kSlack of it leaves the accumulators unscaled.
constexpr float kSlack = 8.0f;

// Chunks of K/V a wave keeps in registers: the one being computed and
// NBUF - 1 in flight behind it.
#ifndef PKV_MFMA_NBUF
#define PKV_MFMA_NBUF 2
#endif
// One-byte caches keep two chunks as well.  Their chunk is half the bytes,
// and three chunks used to serve the 70B-shaped batch better; since the past-
// the-end loads read the idle tiles and the shares follow the dealt
// workgroup order, two are 1-2 % faster on the 8B-shaped int8 and FP8 batches
// and level on the 70B-shaped one (four and six were slower still).
#ifndef PKV_MFMA_NBUF_I8
#define PKV_MFMA_NBUF_I8 2
#endif

// Loads of a buffer past the share's end read these bytes instead of K/V:
// two (block, kv head) tiles of the largest kind (bf16 at D = 128), which
// every wave shares and the L2 keeps, so the steps that finish a group of NB
// cost no HBM reads.  Their values are never used (no token is counted there
// and the V rows are masked), so they are left as loaded: zero.
constexpr int kIdleTileBytes = 32 * 128;
__device__ __align__(4096) uint8_t g_idle_tiles[2 * kIdleTileBytes];

// A plan's walk starts from its record: the wave's share and its first
// chunks' cursors and blocks, read with scalar loads (one round trip, where
// the kernel's own schedule takes the lengths' and then the block table's
// before the first K/V request).  The chunk scan and the lengths come from
// the plan's header as the walk needs them.  Returns false when the wave has
// no work.
template <int W>
__device__ bool plan_begin(const SplitParams &P, ShareT<true> &sh, const int32_t *&rec) {
  const int w = threadIdx.x >> 6;
  sh.wave = uniform((P.wg_dealt ? (int)blockIdx.x : xcd_logical(blockIdx.x, gridDim.x)) * W + w);
  sh.s_incl = P.ws_hdr + PKV_HDR_INTS;
  sh.s_len = P.plan;
  sh.ctx = P.ctx;
  sh.tables = P.tables;
  sh.B = P.B;
  sh.max_blocks = P.max_blocks;
  sh.max_ctx = P.max_ctx;
  sh.num_blocks = P.num_blocks;
  if (sh.wave >= P.plan_cap) return false;  // every wave with work has a record
  rec = P.plan + pkv_plan_lens_ints(P.B) + (size_t)sh.wave * PKV_PLAN_REC_INTS;
  sh.lo = (int64_t)(uint32_t)sload_i32(rec) | ((int64_t)sload_i32(rec + 1) << 32);
  sh.hi = (int64_t)(uint32_t)sload_i32(rec + 2) | ((int64_t)sload_i32(rec + 3) << 32);
  return sh.lo < sh.hi;
}

// Cursor and blocks of a wave's k-th chunk from its plan record.
__device__ __forceinline__ void plan_chunk(const int32_t *rec, int k, Cursor &c, int &pa, int &pb) {
  const int32_t *r = rec + 4 + kPlanCursorInts * k;
  c.b = sload_i32(r);
  c.g = sload_i32(r + 1);
  c.j = sload_i32(r + 2);
  c.cnt = sload_i32(r + 3);
  c.n = sload_i32(r + 4);
  c.seg0 = (int64_t)(uint32_t)sload_i32(r + 5) | ((int64_t)sload_i32(r + 6) << 32);
  pa = sload_i32(r + 7);
  pb = sload_i32(r + 8);
}

// Records wave sh.wave's plan (lane 0): lo and hi of its share, or an empty
// share (WORK false), then the cursors and blocks of its first
// PKV_PLAN_CHUNKS chunks as the self-scheduled prologue located them.  The
// stores are issued before the wave's first loads, so no wait for a load
// is held by them.
template <bool WORK, int NB>
__device__ __forceinline__ void plan_write(const SplitParams &P, const Share &sh, const Cursor *cq, const int *pa,
                                           const int *pb) {
  static_assert(NB >= PKV_PLAN_CHUNKS, "a record holds chunks the prologue has located");
  if ((threadIdx.x & 63) != 0 || sh.wave >= P.plan_cap) return;
  int32_t *rec = P.plan + pkv_plan_lens_ints(P.B) + (size_t)sh.wave * PKV_PLAN_REC_INTS;
  const int64_t lo = WORK ? sh.lo : 0, hi = WORK ? sh.hi : 0;
  *reinterpret_cast<int4 *>(rec) = make_int4((int)(uint32_t)lo, (int)(lo >> 32), (int)(uint32_t)hi, (int)(hi >> 32));
  if constexpr (WORK) {
#pragma unroll
    for (int k = 0; k < PKV_PLAN_CHUNKS; ++k) {
      if (lo + k >= hi) break;
      int32_t *r = rec + 4 + kPlanCursorInts * k;
      *reinterpret_cast<int4 *>(r) = make_int4(cq[k].b, cq[k].g, cq[k].j, cq[k].cnt);
      *reinterpret_cast<int4 *>(r + 4) = make_int4(cq[k].n, (int)(uint32_t)cq[k].seg0, (int)(cq[k].seg0 >> 32), pa[k]);
      r[8] = pb[k];
    }
  }
}

// MODE 0: the kernel computes its schedule (chunk scan of the lengths, then
// each wave's share) and, given a plan buffer (P.plan), records it there;
// MODE 1: it runs from a recorded plan (plan_begin).
template <int D, int W, int NB, bool I8, bool F8, bool NT, int MODE>
__global__ __launch_bounds__(64 * W) void decode_mfma_kernel(SplitParams P) {
  constexpr int NKK = D / 32;  // score MFMAs per 16-row token set
  constexpr int NNN = D / 16;  // PV MFMAs
  constexpr int TB = I8 ? 16 * D + 64 : 32 * D;  // bytes per (block, kv head) tile
  static_assert(TB <= kIdleTileBytes, "the idle tiles must cover a tile");
  // K registers per 16-row token set: one 16-byte unit per score MFMA for
  // bf16; for int8 one unit holds the codes of two MFMAs (16 elements).
  constexpr int NKU = I8 ? NKK / 2 : NKK;
  using VUnit = std::conditional_t<I8, uint2, uint4>;  // 8 elements of V
  extern __shared__ __align__(16) int32_t s_lds[];  // chunk scan, lengths, wave totals

  const int lane = threadIdx.x & 63;
  const int H = P.H, G = P.G;
  const uint32_t t_start = (uint32_t)__builtin_amdgcn_s_memrealtime();
  // Rows of empty sequences are zeroed by the first workgroup: in mode 0
  // within the schedule, in mode 1 here, from the plan's chunk scan, on every
  // exit of each of its waves (each takes its own lanes' sequences).
  auto zero_empty = [&]() {
    if constexpr (MODE == 1) {
      if (blockIdx.x != 0) return;
      const int32_t *incl = P.ws_hdr + PKV_HDR_INTS;
      for (int b = threadIdx.x; b < P.B; b += 64 * W)
        if (incl[b] == (b ? incl[b - 1] : 0)) {
          float *row = P.out + (size_t)b * P.Hq * D;  // out is only 4-byte aligned
          for (int i = 0; i < P.Hq * D; ++i) row[i] = 0.f;
        }
    }
  };
  ShareT<MODE == 1> sh;
  const int32_t *rec = nullptr;
  if constexpr (MODE == 1) {
    if (!plan_begin<W>(P, sh, rec)) {
      zero_empty();
      return;
    }
  } else {
    if (!split_begin<W, D>(P, s_lds, sh)) {
      if (P.plan) plan_write<false, NB>(P, sh, nullptr, nullptr, nullptr);
      return;
    }
  }
  const int64_t lo = sh.lo, hi = sh.hi;
  // This wave's ring of finished pieces, written out after its last load.
  uint8_t *const ring = reinterpret_cast<uint8_t *>(s_lds) + P.ring_off + (threadIdx.x >> 6) * P.nrec * P.rec_bytes;
  int held = 0;  // records in the ring
  // A record: G rows of D floats, G (m, l) pairs, then the piece's place as
  // an int4 at the next 16-byte boundary (G may be odd).
  const int meta_off = (G * D * 4 + G * 8 + 15) & ~15;

  const int r16 = lane & 15, grp = lane >> 4;
  // Row r16 of the score MFMAs holds a token of block (r16 >> 3); see header.
  const int ksel = r16 >> 3;
  const int ktx = ((r16 >> 2) & 1) * 8 + (r16 & 3);
  const int vsel = grp >> 1, vhalf = grp & 1;
  // Element group (8 elements of a row) that lane group grp feeds to score
  // MFMA kk.  Any one-to-one choice gives the same dot products as long as K
  // and Q follow it; int8 pairs the two halves of one 16-byte unit.
  auto kgroup = [&](int kk) { return I8 ? 8 * (kk >> 1) + 2 * grp + (kk & 1) : 4 * kk + grp; };
  const uint8_t *kpool = reinterpret_cast<const uint8_t *>(P.k_pool);
  const uint8_t *vpool = reinterpret_cast<const uint8_t *>(P.v_pool);
  const uint16_t *qbase = reinterpret_cast<const uint16_t *>(P.q);
  // Columns G..15 repeat head G-1: the columns of both products never mix,
  // and those lanes store nothing.  (Their load is not masked: a load under
  // a lane mask would leave the memory counter unknown after it.)
  const int qh = min(r16, G - 1);

  // Per buffer: the chunk's cursor, physical blocks, query slices, K and V.
  // A buffer's query slices are requested when the buffer is located for its
  // chunk, NB steps before their use and right after a step's V requests, and
  // only when that chunk lies in another segment than the slices the buffer
  // holds (qseg).  A wait for a V then covers at most query loads issued
  // with it: query loads placed before a K wait instead would make that wait
  // take a full round trip at every segment start, since the compiler counts
  // the loads in flight on the path without them.
  Cursor cq[NB];
  int pa[NB], pb[NB];
  bf16x8_t qb[NB][NKK];
  int64_t qseg[NB];
  uint4 ax[NB][NKU], ay[NB][NKU];
  VUnit va[NB][NNN];
  float4 ksc[NB][2], vsc[NB][2];  // int8: scales of this lane's 8 token slots

  // The tile of buffer i's first (sel 0) or second block; an idle buffer
  // (pa < 0, past the share's end) reads the shared idle tiles.
  auto tile = [&](const uint8_t *pool, int i, int sel, int g) -> const uint8_t * {
    if (pa[i] < 0) return g_idle_tiles + (sel ? TB : 0);
    return pool + ((size_t)(sel ? pb[i] : pa[i]) * H + g) * TB;
  };
  auto load_q = [&](auto bi) {  // query slices of buffer bi's chunk
    constexpr int I = decltype(bi)::value;
    const Cursor &c = cq[I];
    const uint4 *qr = reinterpret_cast<const uint4 *>(qbase + ((size_t)c.b * P.Hq + (size_t)c.g * G + qh) * D);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint4 u = qr[kgroup(kk)];
      qb[I][kk] = as_bf16x8<F8>(u);
    }
    qseg[I] = c.seg0;
  };
  auto issue = [&](auto bi) {  // K of the chunk held in buffer bi
    constexpr int I = decltype(bi)::value;
    const Cursor &c = cq[I];
    const uint4 *kt = reinterpret_cast<const uint4 *>(tile(kpool, I, ksel, c.g));
#pragma unroll
    for (int ku = 0; ku < NKU; ++ku) {
      // 16-byte unit of the lane's token row: int8 unit 4ku+grp holds the
      // element groups 2(4ku+grp) and +1 of score MFMAs 2ku and 2ku+1.
      const int cu = 4 * ku + grp;
      ax[I][ku] = load_u4<NT>(kt + cu * 16 + (I8 ? k8_unit(ktx) : ktx));
      ay[I][ku] = load_u4<NT>(kt + cu * 16 + (I8 ? k8_unit(ktx + 4) : ktx + 4));
    }
    if constexpr (I8) {
      const float4 *sc = reinterpret_cast<const float4 *>(tile(kpool, I, vsel, c.g) + 16 * D + 32 * vhalf);
      ksc[I][0] = load_f4<NT>(sc);
      ksc[I][1] = load_f4<NT>(sc + 1);
    }
  };
  auto issue_v = [&](auto bi) {
    constexpr int I = decltype(bi)::value;
    const uint8_t *vt = tile(vpool, I, vsel, cq[I].g);
    if constexpr (I8) {
#pragma unroll
      for (int nn = 0; nn < NNN; ++nn) va[I][nn] = load_u2<NT>(vt + (16 * nn + r16) * 16 + 8 * vhalf);
      const float4 *sc = reinterpret_cast<const float4 *>(vt + 16 * D + 32 * vhalf);
      vsc[I][0] = load_f4<NT>(sc);
      vsc[I][1] = load_f4<NT>(sc + 1);
    } else {
      const uint4 *u = reinterpret_cast<const uint4 *>(vt);
#pragma unroll
      for (int nn = 0; nn < NNN; ++nn) va[I][nn] = load_u4<NT>(u + 2 * (16 * nn + r16) + vhalf);
    }
  };

  f32x4_t o[NNN];
#pragma unroll
  for (int nn = 0; nn < NNN; ++nn) o[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  // Every load is issued whatever the share's length: a buffer past the
  // share's end takes the last real chunk's cursor and reads the idle tiles
  // for K/V (its query registers keep what they hold; no token of an idle
  // step is counted).  Loads issued on some paths only would
  // leave the count of loads in flight unknown, and the waits would then
  // drain every buffer each step.
  auto idle_after = [&](int to, int from) {
    cq[to] = cq[from];
    pa[to] = -1;
    pb[to] = -1;
  };
  // Prologue: chunks lo .. lo+NB-2 are requested, chunk lo+NB-1 located.
  auto locate_first = [&](auto bi) {  // chunk lo + bi of the share, which exists
    constexpr int I = decltype(bi)::value;
    if constexpr (MODE == 1 && I < PKV_PLAN_CHUNKS) {
      plan_chunk(rec, I, cq[I], pa[I], pb[I]);
    } else if constexpr (I == 0) {
      cq[0] = sh.first();
      sh.blocks(cq[0], pa[0], pb[0]);
    } else {
      cq[I] = sh.next(cq[I > 0 ? I - 1 : 0]);
      sh.blocks(cq[I], pa[I], pb[I]);
    }
  };
  locate_first(std::integral_constant<int, 0>{});
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    ((Is == 0 ? (void)0
              : (lo + Is < hi ? locate_first(std::integral_constant<int, Is>{}) : idle_after(Is, Is - 1))), ...);
  }(std::make_integer_sequence<int, NB>{});
  if constexpr (MODE == 0)
    if (P.plan) plan_write<true, NB>(P, sh, cq, pa, pb);
  // Requests leave in the order the loop issues them (every buffer's query
  // slices first, then K and V of each chunk): waits at the loop head are
  // counted over all of them, and a prologue that sent a chunk's K last
  // would make the first of them wait for everything.
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    (load_q(std::integral_constant<int, Is>{}), ...);
  }(std::make_integer_sequence<int, NB>{});
  __builtin_amdgcn_sched_barrier(0);
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    ((Is < NB - 1 ? (issue(std::integral_constant<int, Is>{}), __builtin_amdgcn_sched_barrier(0),
                     issue_v(std::integral_constant<int, Is>{}), __builtin_amdgcn_sched_barrier(0))
                  : (void)0),
     ...);
  }(std::make_integer_sequence<int, NB>{});

  int64_t x = lo;
  // One step computes chunk x from buffer I, requests chunk x+NB-1 into the
  // buffer chunk x-1 used, and locates chunk x+NB into buffer I.
  auto step = [&](auto bi) {
    constexpr int I = decltype(bi)::value;
    constexpr int J = (I + NB - 1) % NB;
    f32x4_t sx = {0.f, 0.f, 0.f, 0.f}, sy = {0.f, 0.f, 0.f, 0.f};
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
      sx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kx, qb[I][kk], sx, 0, 0, 0);
      sy = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ky, qb[I][kk], sy, 0, 0, 0);
    }
    if (x + NB - 1 >= hi) idle_after(J, I);  // no chunk x + NB - 1 in the share
    issue(std::integral_constant<int, J>{});

    const Cursor &cur = cq[I];
    // Past the share's end the loop runs on to the end of its group of NB
    // steps over the idle tiles with no token counted: nothing is stored,
    // and the loop keeps one exit, after a whole group.
    const bool real = x < hi;
    const int n = real ? cur.n : 0;
    const int tok0 = 32 * cur.j;
    const int tb = tok0 + 16 * vsel + 8 * vhalf;  // this lane's first token (scores and V)
    float s[8];
    if constexpr (I8) {
      const float ks[8] = {ksc[I][0].x, ksc[I][0].y, ksc[I][0].z, ksc[I][0].w,
                           ksc[I][1].x, ksc[I][1].y, ksc[I][1].z, ksc[I][1].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[r] = (tb + r < n) ? sx[r] * ks[r] * P.scale_log2 : -INFINITY;
        s[4 + r] = (tb + 4 + r < n) ? sy[r] * ks[4 + r] * P.scale_log2 : -INFINITY;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[r] = (tb + r < n) ? sx[r] * P.scale_log2 : -INFINITY;
        s[4 + r] = (tb + 4 + r < n) ? sy[r] * P.scale_log2 : -INFINITY;
      }
    }
    float cmax = s[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) cmax = fmaxf(cmax, s[r]);
    cmax = rows_max4_swap(cmax);
    // The reference maximum moves only when some head's scores pass it by
    // more than kSlack (base 2), and then for the whole wave at once: weights
    // stay below 2^kSlack, and most chunks skip rescaling the accumulators.
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(cmax > m + kSlack) != 0, 0)) {
      const float mnew = fmaxf(m, cmax);
      const float alpha = fast_exp2(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int nn = 0; nn < NNN; ++nn) o[nn] *= alpha;
    }
    bf16x8_t pv;
    float psum = 0.f;
    if constexpr (I8) {
      const float vs[8] = {vsc[I][0].x, vsc[I][0].y, vsc[I][0].z, vsc[I][0].w,
                           vsc[I][1].x, vsc[I][1].y, vsc[I][1].z, vsc[I][1].w};
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float e = fast_exp2(s[r] - m);
        psum += e;
        pv[r] = (__bf16)((tb + r < n) ? e * vs[r] : 0.f);  // scales past the context may be NaN
      }
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const __bf16 pr = (__bf16)fast_exp2(s[r] - m);
        pv[r] = pr;
        psum += (float)pr;  // the PV numerator uses the rounded weights too
      }
    }
    l += psum;
    if constexpr (!I8 || F8) {
      if (tok0 + 32 > n) {  // slots past the context may hold anything, NaN included
        const int nvalid = min(max(n - tb, 0), 8);
#pragma unroll
        for (int nn = 0; nn < NNN; ++nn) va[I][nn] = keep_first(va[I][nn], nvalid);
      }
    }
#pragma unroll
    for (int nn = 0; nn < NNN; ++nn) o[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8<F8>(va[I][nn]), pv, o[nn], 0, 0, 0);
    issue_v(std::integral_constant<int, J>{});

    if (real && (x + 1 >= hi || cur.j == cur.cnt - 1)) {  // the piece ends here
      const float lsum = rows_sum4(l);
      const bool whole = sh.whole(cur);
      const int slot = whole ? 0 : sh.slot(cur, P.nslots);
      if (held < P.nrec) {
        // The piece's rows go to the wave's LDS ring and reach memory after
        // the wave's last load: LDS traffic has a counter of its own, so the
        // K/V loads in flight keep flowing.
        uint8_t *rec = ring + held * P.rec_bytes;
        if (r16 < G) {
          const float inv = whole ? 1.f / lsum : 1.f;
          float *row = reinterpret_cast<float *>(rec) + r16 * D + 4 * grp;
#pragma unroll
          for (int nn = 0; nn < NNN; ++nn)
            *reinterpret_cast<float4 *>(row + 16 * nn) =
                make_float4(o[nn][0] * inv, o[nn][1] * inv, o[nn][2] * inv, o[nn][3] * inv);
          if (grp == 0) *reinterpret_cast<float2 *>(rec + G * D * 4 + r16 * 8) = make_float2(m, lsum);
        }
        if (lane == 0) *reinterpret_cast<int4 *>(rec + meta_off) = make_int4(whole, cur.b, cur.g, slot);
        ++held;
      } else {
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
            const size_t ps = (size_t)slot * G + r16;
            float *dst = P.ws_o + ps * D + 4 * grp;
#pragma unroll
            for (int nn = 0; nn < NNN; ++nn)
              *reinterpret_cast<float4 *>(dst + 16 * nn) = make_float4(o[nn][0], o[nn][1], o[nn][2], o[nn][3]);
            if (grp == 0) *reinterpret_cast<float2 *>(P.ws_ml + 2 * ps) = make_float2(m, lsum);
          }
        }
        // Stores share the memory counter with loads: drain it here, so that
        // the loads in flight are counted exactly on every path (otherwise
        // each chunk's waits would assume the worst and drain it).
        __builtin_amdgcn_s_waitcnt(kDrainVm);
      }
#pragma unroll
      for (int nn = 0; nn < NNN; ++nn) o[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m = -INFINITY;
      l = 0.f;
    }
    if (x + NB < hi) {
      cq[I] = sh.next(cq[J]);
      sh.blocks(cq[I], pa[I], pb[I]);
      if (cq[I].seg0 != qseg[I]) load_q(std::integral_constant<int, I>{});
    }
    ++x;
  };
  while (x < hi) {
    [&]<int... Is>(std::integer_sequence<int, Is...>) {
      (step(std::integral_constant<int, Is>{}), ...);
    }(std::make_integer_sequence<int, NB>{});
  }
  // Write out the ring: G rows of D floats per record, 16 bytes per lane,
  // then the (m, l) of a partial.
  for (int r = 0; r < held; ++r) {
    const uint8_t *rec = ring + r * P.rec_bytes;
    const int4 meta = *reinterpret_cast<const int4 *>(rec + meta_off);
    const bool whole = uniform(meta.x) != 0;
    const size_t row0 = (size_t)uniform(meta.y) * P.Hq + (size_t)uniform(meta.z) * G;
    const int slot = uniform(meta.w);
    for (int u = lane; u < G * (D / 4); u += 64) {
      const int h = u / (D / 4), c = 4 * (u % (D / 4));
      const float4 v = *reinterpret_cast<const float4 *>(rec + (h * D + c) * 4);
      float *dst = whole ? P.out + (row0 + h) * D + c : P.ws_o + ((size_t)slot * G + h) * D + c;
      *reinterpret_cast<float4 *>(dst) = v;
    }
    if (!whole && lane < G)
      *reinterpret_cast<float2 *>(P.ws_ml + 2 * ((size_t)slot * G + lane)) =
          *reinterpret_cast<const float2 *>(rec + G * D * 4 + lane * 8);
  }
  zero_empty();
  // Optional trace: the wave's XCD group (workgroups are dealt round-robin
  // to the 8 XCDs), its chunks, and its start and end times (100 MHz clock,
  // low 32 bits), from which per-XCD streaming rates and weights follow.
  if (P.trace && lane == 0 && sh.wave < PKV_TRACE_WAVES) {
    const uint32_t t_end = (uint32_t)__builtin_amdgcn_s_memrealtime();
    *reinterpret_cast<int4 *>(P.trace + PKV_TRACE_INTS * sh.wave) =
        make_int4((int)(blockIdx.x & 7), (int)(hi - lo), (int)t_start, (int)t_end);
  }
}

#ifndef PKV_MFMA_WAVES
#define PKV_MFMA_WAVES 4
#endif
constexpr int kWaves = PKV_MFMA_WAVES;
// LDS a workgroup may take, result rings included: one workgroup per CU
// (over half of the 160 KiB), or two.
constexpr size_t kRingLdsOneWg = 96 * 1024;
constexpr size_t kRingLdsTwoWg = 64 * 1024;
// Records a wave ring holds at most.
constexpr size_t kMaxRecords = 16;

// I8: one-byte codes (int8, or FP8 E4M3 when F8) with per-row scales.
template <int D, bool I8, bool F8, bool NT>
int launch(const pkv_decode_args &a, const SplitParams &p0) {
  constexpr int NB = I8 ? PKV_MFMA_NBUF_I8 : PKV_MFMA_NBUF;
  // The grid is the one of the self-scheduling kernel in both modes, so that
  // a plan and the calls that run from it agree on every wave's share.
  auto kern = decode_mfma_kernel<D, kWaves, NB, I8, F8, NT, 0>;
  SplitParams p = p0;
  // A one-byte (block, kv head) tile is 2112 bytes, so every other tile
  // shares a 128-byte line with the next kv head's tile.  The waves reading
  // kv heads g and g + 1 at the same list position are 1/8 of the grid
  // apart: as dealt to the XCDs (round robin) they sit on one XCD and that
  // line comes from HBM once; renumbered into contiguous eighths they sit on
  // two XCDs and it is fetched twice (3 % of the bytes).  Batches of shared
  // blocks (two waves per SIMD) and per-XCD weights keep the eighths.
  bool weighted = false;
  for (int i = 0; i < PKV_REGIONS; ++i) weighted |= a.xw[i] != 0;
  p.wg_dealt = I8 && a.waves_per_simd == 1 && !weighted;
  const size_t split = pkv_split_lds_bytes(a.num_seqs, kWaves);
  // Result rings: what LDS is left of the workgroup's share of the CU, split
  // over its waves, in records of G rows of D floats, G (m, l) pairs and the
  // piece's place, 16-byte aligned.
  const int G = a.num_q_heads / a.L->num_kv_heads;
  const int rec = ((G * D * 4 + G * 8 + 15) & ~15) + 16;
  const size_t budget = a.waves_per_simd == 1 ? kRingLdsOneWg : kRingLdsTwoWg;
  p.ring_off = (int32_t)split;
  p.rec_bytes = rec;
  p.nrec = budget > split ? (int32_t)std::min<size_t>((budget - split) / kWaves / rec, kMaxRecords) : 0;
  size_t lds = split + (size_t)kWaves * p.nrec * rec;
  // One wave per SIMD: a workgroup takes more than half of a CU's 160 KiB of
  // LDS, so no second one is placed beside it.  Two waves on one SIMD do not
  // progress alike (the older wins issue), which leaves the younger behind.
  if (a.waves_per_simd == 1) lds = std::max<size_t>(lds, PKV_LDS_ONE_WG_PER_CU);
  int nwg = 0;
  if (int rc = pkv_split_grid(reinterpret_cast<const void *>(kern), 64 * kWaves, lds, a, &nwg)) return rc;
  const hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  if (a.plan_mode == 1) {
    // Runs on the grid above, that of the call that recorded the plan (the
    // call below only sets the kernel's LDS limit).
    auto kp = decode_mfma_kernel<D, kWaves, NB, I8, F8, NT, 1>;
    int unused = 0;
    if (int rc = pkv_split_grid(reinterpret_cast<const void *>(kp), 64 * kWaves, lds, a, &unused)) return rc;
    hipLaunchKernelGGL(kp, dim3(nwg), dim3(64 * kWaves), lds, st, p);
    return (int)hipGetLastError();
  }
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(64 * kWaves), lds, st, p);
  return (int)hipGetLastError();
}

template <bool I8, bool F8, bool NT>
int launch_d(const pkv_decode_args &a, const SplitParams &p) {
  return a.L->head_dim == 128 ? launch<128, I8, F8, NT>(a, p) : launch<64, I8, F8, NT>(a, p);
}

template <bool NT>
int launch_t(const pkv_decode_args &a, const SplitParams &p) {
  if (a.L->kv_dtype == PKV_INT8) return launch_d<true, false, NT>(a, p);
  if (a.L->kv_dtype == PKV_FP8) return launch_d<true, true, NT>(a, p);
  return launch_d<false, false, NT>(a, p);
}

}  // namespace

int pkv_launch_decode_mfma(const pkv_decode_args &a) {
  const SplitParams p = pkv_split_params(a);
  return a.streaming ? launch_t<true>(a, p) : launch_t<false>(a, p);
}
