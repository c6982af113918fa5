// Streaming-read probe: how fast one MI355X reads a buffer of 4 KiB tiles in
// a given order, with the access pattern of the decode kernels.  It computes
// nothing of the method; it gives the achievable HBM read rate that the decode
// kernels' rate is compared with (paged decode reads random 4 KiB (block, kv
// head) tiles through the block tables).
//
// Grid and pattern as the decode kernels run them: one 256-thread workgroup
// per compute unit (dynamic LDS above half of the CU's 160 KiB keeps a second
// one away), every wave an equal contiguous share of the tile order, four
// tiles (16 KiB, a decode chunk's K and V) per step, every lane 16-byte loads,
// two steps of loads kept in registers (one in flight while the other is
// folded), as the bf16 decode kernel keeps two chunks.  Optionally two
// workgroups per compute unit (two waves per SIMD) keep twice the bytes in
// flight, and the loads carry the non-temporal hint (streamed through the
// caches, as the decode kernels read tiles that are used once).  The words read are folded with xor
// into one value per wave, stored at the end, so no load is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace {

constexpr int kWaves = 4;
constexpr int kTilesPerStep = 4;
constexpr int kTileUnits = 4096 / 16 / 64;  // 16-byte loads per lane per tile
constexpr int kLdsOneWgPerCu = 81 * 1024;

typedef const int32_t __attribute__((address_space(4))) *const_i32;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NB = 2;

template <bool NT>
__global__ __launch_bounds__(64 * kWaves) void stream_tiles_kernel(const uint4 *buf, int64_t n_steps,
                                                                   const int32_t *order, uint32_t *sink) {
  const int64_t n_tiles = n_steps * kTilesPerStep;
  extern __shared__ int32_t s_unused[];
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  // The wave index is uniform: tile ids then come through scalar loads and
  // never wait behind the tile data.
  const int64_t w = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWaves + (threadIdx.x >> 6)));
  const int64_t lo = w * n_steps / nw, hi = (w + 1) * n_steps / nw;
  if (lo >= hi) return;
  uint4 r[NB][kTilesPerStep][kTileUnits];
  // Loads of step x into buffer I; a step past the share re-reads the last
  // one, so every path issues the same loads and the waits stay exact.
  auto issue = [&](auto bi, int64_t x) {
    constexpr int I = decltype(bi)::value;
    const int64_t s = x < hi ? x : hi - 1;
#pragma unroll
    for (int t = 0; t < kTilesPerStep; ++t) {
      int64_t tile = *(const_i32)(order + s * kTilesPerStep + t);
      tile = tile < 0 ? 0 : tile >= n_tiles ? n_tiles - 1 : tile;  // a bad order cannot leave the buffer
      const uint4 *p = buf + (size_t)tile * (4096 / 16);
#pragma unroll
      for (int u = 0; u < kTileUnits; ++u) {
        if constexpr (NT) {
          const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + 64 * u + lane));
          r[I][t][u] = make_uint4(v.x, v.y, v.z, v.w);
        } else {
          r[I][t][u] = p[64 * u + lane];
        }
      }
    }
  };
  uint32_t acc = 0;
  auto fold = [&](auto bi) {
    constexpr int I = decltype(bi)::value;
#pragma unroll
    for (int t = 0; t < kTilesPerStep; ++t)
#pragma unroll
      for (int u = 0; u < kTileUnits; ++u) acc ^= r[I][t][u].x ^ r[I][t][u].y ^ r[I][t][u].z ^ r[I][t][u].w;
  };
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    ((issue(std::integral_constant<int, Is>{}, lo + Is), __builtin_amdgcn_sched_barrier(0)), ...);
  }(std::make_integer_sequence<int, NB>{});
  // Each step folds the oldest buffer and refills it with the step NB ahead,
  // so NB - 1 steps of loads stay in flight behind the one being folded.
  int64_t x = lo;
  while (x < hi) {
    [&]<int... Is>(std::integer_sequence<int, Is...>) {
      ((fold(std::integral_constant<int, Is>{}), __builtin_amdgcn_sched_barrier(0),
        issue(std::integral_constant<int, Is>{}, x + NB), __builtin_amdgcn_sched_barrier(0), ++x),
       ...);
    }(std::make_integer_sequence<int, NB>{});
  }
  acc ^= __shfl_xor(acc, 1, 64);
  if (lane == 0) sink[w] = acc;
}

// Fixed cost of a launch: an empty kernel on the decode kernels' grid (one
// 256-thread workgroup per compute unit, LDS above half of the CU) whose
// waves record their first and last clock (s_memrealtime, 100 MHz).  The
// time events on the stream see around it, less the span of its waves, is
// what a launch costs beside the work of its waves.
__global__ __launch_bounds__(64 * kWaves) void launch_cost_kernel(uint32_t *clock) {
  extern __shared__ int32_t s_unused[];
  const uint32_t t0 = (uint32_t)__builtin_amdgcn_s_memrealtime();
  const int w = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const uint32_t t1 = (uint32_t)__builtin_amdgcn_s_memrealtime();
  if ((threadIdx.x & 63) == 0) *reinterpret_cast<uint2 *>(clock + 2 * w) = make_uint2(t0, t1);
}

// Matrix-core issue probe: per iteration, 24 v_mfma_f32_16x16x32_bf16 on
// independent accumulators and/or the vector work that weighs 24 scores
// (fma, base-2 exponential, bf16 pack), with one or two waves per SIMD.
// MODE 0: products only; 1: vector work only; 2: both in program order; 3:
// both, one product then two vector instructions (scheduling groups); 4: 12
// v_mfma_f32_32x32x16_bf16 (the same flops) on independent accumulators.
// The results are folded into one store per lane, so no work is dead.
typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x4_p __attribute__((ext_vector_type(4)));
typedef float f32x2_p __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_p __attribute__((ext_vector_type(2)));

template <int MODE>
__global__ __launch_bounds__(64 * kWaves) void mfma_issue_kernel(const float *in, float *out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8_p a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)in[lane + i];
    b[i] = (__bf16)in[lane + 8 + i];
  }
  f32x4_p acc[24];
  float e[24];
#pragma unroll
  for (int i = 0; i < 24; ++i) {
    acc[i] = f32x4_p{0.f, 0.f, 0.f, 0.f};
    e[i] = in[lane + i];
  }
  uint32_t pk = 0;
  const float m = in[0], mul = in[1];
  typedef float f32x16_p __attribute__((ext_vector_type(16)));
  f32x16_p acc32[MODE == 4 ? 12 : 1];
#pragma unroll
  for (int i = 0; i < (MODE == 4 ? 12 : 1); ++i) acc32[i] = f32x16_p{};
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == 4) {
#pragma unroll
      for (int i = 0; i < 12; ++i) acc32[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc32[i], 0, 0, 0);
    } else if constexpr (MODE != 1) {
#pragma unroll
      for (int i = 0; i < 24; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
    }
    if constexpr (MODE >= 1 && MODE <= 3) {
#pragma unroll
      for (int i = 0; i < 24; ++i) e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(e[i], mul, -m));
#pragma unroll
      for (int i = 0; i < 24; i += 2)
        pk ^= __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_p{e[i], e[i + 1]}, bf16x2_p));
    }
    if constexpr (MODE == 3) {
#pragma unroll
      for (int i = 0; i < 24; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
    }
  }
  float r = (float)pk;
#pragma unroll
  for (int i = 0; i < 24; ++i) r += acc[i][0] + acc[i][3] + e[i];
  if constexpr (MODE == 4) {
#pragma unroll
    for (int i = 0; i < 12; ++i) r += acc32[i][0] + acc32[i][15];
  }
  out[blockIdx.x * (64 * kWaves) + threadIdx.x] = r;
}

// Load-pattern probe: the decode kernels' per-lane loads of one 32-token
// chunk (two (block, kv head) tiles of K and of V, named by a random order),
// with no arithmetic, so that a layout or load choice is measured apart from
// the kernel's work.  B1 = false: bf16 tiles (4 KiB), 8 x 16 B of K and 8 x 16
// B of V per lane; B1 = true: one-byte tiles (2112 B: codes, then scales), 4
// x 16 B of K, 2 x 16 B of K scales, 8 x 8 B of V, 2 x 16 B of V scales.
// VARIANT bit 0: K loads on whole 128-byte lines (the two loads of a 16-byte
// unit row take slots 0-7 and 8-15) instead of the score products' halves
// ({0-3, 8-11} and {4-7, 12-15}); bit 1: no query slices (otherwise 4 x 16 B
// per lane from a 256 KiB buffer that stays in L2, as a kernel reloading them
// with every chunk).  Two chunks of loads in registers, as the kernels keep.
template <bool NT> __device__ __forceinline__ uint4 pload16(const uint8_t *p) {
  if constexpr (NT) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *reinterpret_cast<const uint4 *>(p);
  }
}
template <bool NT> __device__ __forceinline__ uint2 pload8(const uint8_t *p) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (NT) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    return make_uint2(v.x, v.y);
  } else {
    return *reinterpret_cast<const uint2 *>(p);
  }
}

template <bool NT, bool B1, int VARIANT>
__global__ __launch_bounds__(64 * kWaves) void load_pattern_kernel(const uint8_t *kp, const uint8_t *vp,
                                                                   const uint8_t *qb, int64_t n_chunks,
                                                                   const int32_t *order, uint32_t *sink) {
  constexpr int TB = B1 ? 2112 : 4096;
  constexpr int NKU = B1 ? 2 : 4;
  constexpr bool WHOLE = VARIANT & 1, NOQ = VARIANT & 2;
  extern __shared__ int32_t s_unused[];
  const int64_t n_tiles = 2 * n_chunks;
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * kWaves;
  const int64_t w = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWaves + (threadIdx.x >> 6)));
  const int64_t lo = w * n_chunks / nw, hi = (w + 1) * n_chunks / nw;
  if (lo >= hi) return;
  const int r16 = lane & 15, grp = lane >> 4, ksel = r16 >> 3, vsel = grp >> 1, vhalf = grp & 1;
  const int ktx = ((r16 >> 2) & 1) * 8 + (r16 & 3);
  const int ka = WHOLE ? (r16 & 7) : ktx, kb = WHOLE ? 8 + (r16 & 7) : ktx + 4;
  uint4 q[NB][4], ax[NB][NKU], ay[NB][NKU], sc[NB][4], vw[NB][8];
  uint2 vn[NB][8];
  auto issue = [&](auto bi, int64_t x) {
    constexpr int I = decltype(bi)::value;
    const int64_t s = x < hi ? x : hi - 1;
    int64_t t0 = *(const_i32)(order + 2 * s), t1 = *(const_i32)(order + 2 * s + 1);
    t0 = t0 < 0 ? 0 : t0 >= n_tiles ? n_tiles - 1 : t0;  // a bad order cannot leave the pools
    t1 = t1 < 0 ? 0 : t1 >= n_tiles ? n_tiles - 1 : t1;
    if constexpr (!NOQ) {
      const uint8_t *qr = qb + ((w & 255) * 4 + (r16 < 3 ? r16 : 3)) * 256;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        q[I][kk] = pload16<false>(qr + 16 * (B1 ? 8 * (kk >> 1) + 2 * grp + (kk & 1) : 4 * kk + grp));
    }
    const uint8_t *kt = kp + (size_t)(ksel ? t1 : t0) * TB;
#pragma unroll
    for (int ku = 0; ku < NKU; ++ku) {
      const int cu = 4 * ku + grp;
      ax[I][ku] = pload16<NT>(kt + 16 * (cu * 16 + ka));
      ay[I][ku] = pload16<NT>(kt + 16 * (cu * 16 + kb));
    }
    const uint8_t *kst = kp + (size_t)(vsel ? t1 : t0) * TB;
    const uint8_t *vt = vp + (size_t)(vsel ? t1 : t0) * TB;
    if constexpr (B1) {
      sc[I][0] = pload16<NT>(kst + 2048 + 32 * vhalf);
      sc[I][1] = pload16<NT>(kst + 2048 + 32 * vhalf + 16);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) vn[I][nn] = pload8<NT>(vt + (16 * nn + r16) * 16 + 8 * vhalf);
      sc[I][2] = pload16<NT>(vt + 2048 + 32 * vhalf);
      sc[I][3] = pload16<NT>(vt + 2048 + 32 * vhalf + 16);
    } else {
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) vw[I][nn] = pload16<NT>(vt + 16 * (2 * (16 * nn + r16) + vhalf));
    }
  };
  uint32_t acc = 0;
  auto x4 = [](uint4 u) { return u.x ^ u.y ^ u.z ^ u.w; };
  auto fold = [&](auto bi) {
    constexpr int I = decltype(bi)::value;
    if constexpr (!NOQ)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc ^= x4(q[I][kk]);
#pragma unroll
    for (int ku = 0; ku < NKU; ++ku) acc ^= x4(ax[I][ku]) ^ x4(ay[I][ku]);
    if constexpr (B1) {
#pragma unroll
      for (int k = 0; k < 4; ++k) acc ^= x4(sc[I][k]);
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) acc ^= vn[I][nn].x ^ vn[I][nn].y;
    } else {
#pragma unroll
      for (int nn = 0; nn < 8; ++nn) acc ^= x4(vw[I][nn]);
    }
  };
  [&]<int... Is>(std::integer_sequence<int, Is...>) {
    ((issue(std::integral_constant<int, Is>{}, lo + Is), __builtin_amdgcn_sched_barrier(0)), ...);
  }(std::make_integer_sequence<int, NB>{});
  int64_t x = lo;
  while (x < hi) {
    [&]<int... Is>(std::integer_sequence<int, Is...>) {
      ((fold(std::integral_constant<int, Is>{}), __builtin_amdgcn_sched_barrier(0),
        issue(std::integral_constant<int, Is>{}, x + NB), __builtin_amdgcn_sched_barrier(0), ++x),
       ...);
    }(std::make_integer_sequence<int, NB>{});
  }
  acc ^= __shfl_xor(acc, 1, 64);
  if (lane == 0) sink[w] = acc;
}

template <bool NT, bool B1, int VARIANT>
int launch_pattern(const uint8_t *kp, const uint8_t *vp, const uint8_t *qb, int64_t n_chunks, const int32_t *order,
                   uint32_t *sink, int nwg, hipStream_t stream) {
  auto kern = load_pattern_kernel<NT, B1, VARIANT>;
  if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, kLdsOneWgPerCu))
    return (int)e;
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(64 * kWaves), kLdsOneWgPerCu, stream, kp, vp, qb, n_chunks, order, sink);
  return (int)hipGetLastError();
}

template <bool NT, bool B1>
int launch_pattern_v(int variant, const uint8_t *kp, const uint8_t *vp, const uint8_t *qb, int64_t n_chunks,
                     const int32_t *order, uint32_t *sink, int nwg, hipStream_t stream) {
  switch (variant) {
    case 0: return launch_pattern<NT, B1, 0>(kp, vp, qb, n_chunks, order, sink, nwg, stream);
    case 1: return launch_pattern<NT, B1, 1>(kp, vp, qb, n_chunks, order, sink, nwg, stream);
    case 2: return launch_pattern<NT, B1, 2>(kp, vp, qb, n_chunks, order, sink, nwg, stream);
    default: return launch_pattern<NT, B1, 3>(kp, vp, qb, n_chunks, order, sink, nwg, stream);
  }
}

template <bool NT>
int launch(const void *buf, int64_t n_tiles, const int32_t *order, uint32_t *sink, int nwg, size_t lds,
           hipStream_t stream) {
  auto kern = stream_tiles_kernel<NT>;
  if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, kLdsOneWgPerCu))
    return (int)e;
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(64 * kWaves), lds, stream, reinterpret_cast<const uint4 *>(buf),
                     n_tiles / kTilesPerStep, order, sink);
  return (int)hipGetLastError();
}

}  // namespace

// Read the n_tiles 4 KiB tiles of buf in the order d_order (int32, n_tiles
// entries, each in [0, n_tiles)) on waves_per_simd (1 or 2) workgroups of
// four waves per compute unit, with cached (streaming = 0) or non-temporal
// (streaming = 1) loads.  d_sink receives one uint32 per wave
// (4 * waves_per_simd * compute units of them).  n_tiles must be a positive
// multiple of 4.  Returns a HIP error code (0 = launched), or -1 for bad
// arguments.
extern "C" int pkv_probe_stream_tiles(const void *buf, int64_t n_tiles, const int32_t *d_order,
                                      int32_t waves_per_simd, int32_t streaming, uint32_t *d_sink, void *stream) {
  if (!buf || !d_order || !d_sink || n_tiles <= 0 || n_tiles % kTilesPerStep) return -1;
  if ((waves_per_simd != 1 && waves_per_simd != 2) || (streaming != 0 && streaming != 1)) return -1;
  int dev = 0, cus = 0;
  if (hipError_t e = hipGetDevice(&dev)) return (int)e;
  if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) return (int)e;
  const size_t lds = waves_per_simd == 1 ? kLdsOneWgPerCu : 0;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return streaming ? launch<true>(buf, n_tiles, d_order, d_sink, cus * waves_per_simd, lds, s)
                   : launch<false>(buf, n_tiles, d_order, d_sink, cus * waves_per_simd, lds, s);
}

// One launch of the load-pattern probe (see load_pattern_kernel) on one
// workgroup of four waves per compute unit.  one_byte: 0 bf16 tiles of 4096
// bytes, 1 one-byte tiles of 2112 bytes; variant 0..3 (bit 0 whole-line K,
// bit 1 no query slices); streaming: 0 cached, 1 non-temporal K/V loads.
// d_k and d_v hold 2 * n_chunks tiles each, d_q 256 KiB, d_order 2 * n_chunks
// int32 tile ids in [0, 2 * n_chunks); d_sink one uint32 per wave (4 per
// compute unit).  Returns a HIP error code (0 = launched), or -1 for bad
// arguments.
extern "C" int pkv_probe_load_pattern(int32_t one_byte, int32_t variant, int32_t streaming, const void *d_k,
                                      const void *d_v, const void *d_q, int64_t n_chunks, const int32_t *d_order,
                                      uint32_t *d_sink, void *stream) {
  if (!d_k || !d_v || !d_q || !d_order || !d_sink || n_chunks <= 0 || variant < 0 || variant > 3 ||
      (one_byte != 0 && one_byte != 1) || (streaming != 0 && streaming != 1))
    return -1;
  int dev = 0, cus = 0;
  if (hipError_t e = hipGetDevice(&dev)) return (int)e;
  if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) return (int)e;
  const uint8_t *k = static_cast<const uint8_t *>(d_k), *v = static_cast<const uint8_t *>(d_v),
                *q = static_cast<const uint8_t *>(d_q);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (one_byte)
    return streaming ? launch_pattern_v<true, true>(variant, k, v, q, n_chunks, d_order, d_sink, cus, s)
                     : launch_pattern_v<false, true>(variant, k, v, q, n_chunks, d_order, d_sink, cus, s);
  return streaming ? launch_pattern_v<true, false>(variant, k, v, q, n_chunks, d_order, d_sink, cus, s)
                   : launch_pattern_v<false, false>(variant, k, v, q, n_chunks, d_order, d_sink, cus, s);
}

// One launch of the empty kernel on one workgroup of four waves per compute
// unit; d_clock receives each wave's first and last clock (2 uint32 per
// wave, 8 per compute unit).  Returns a HIP error code (0 = launched), or -1
// for a null d_clock.
extern "C" int pkv_probe_launch_cost(uint32_t *d_clock, void *stream) {
  if (!d_clock) return -1;
  int dev = 0, cus = 0;
  if (hipError_t e = hipGetDevice(&dev)) return (int)e;
  if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) return (int)e;
  if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(launch_cost_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, kLdsOneWgPerCu))
    return (int)e;
  hipLaunchKernelGGL(launch_cost_kernel, dim3(cus), dim3(64 * kWaves), kLdsOneWgPerCu,
                     reinterpret_cast<hipStream_t>(stream), d_clock);
  return (int)hipGetLastError();
}

// One launch of the matrix-core issue probe (mode 0..4, see above) for iters
// iterations on waves_per_simd (1 or 2) workgroups of four waves per compute
// unit.  d_in: 96 floats of input (any finite values); d_out: one float per
// thread (256 * waves_per_simd * compute units).  Returns a HIP error code
// (0 = launched), or -1 for bad arguments.
extern "C" int pkv_probe_mfma_issue(int32_t mode, int32_t waves_per_simd, int32_t iters, const float *d_in,
                                    float *d_out, void *stream) {
  if (!d_in || !d_out || iters <= 0 || mode < 0 || mode > 4 || (waves_per_simd != 1 && waves_per_simd != 2))
    return -1;
  int dev = 0, cus = 0;
  if (hipError_t e = hipGetDevice(&dev)) return (int)e;
  if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) return (int)e;
  const dim3 grid(cus * waves_per_simd), block(64 * kWaves);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: hipLaunchKernelGGL(mfma_issue_kernel<0>, grid, block, 0, s, d_in, d_out, iters); break;
    case 1: hipLaunchKernelGGL(mfma_issue_kernel<1>, grid, block, 0, s, d_in, d_out, iters); break;
    case 2: hipLaunchKernelGGL(mfma_issue_kernel<2>, grid, block, 0, s, d_in, d_out, iters); break;
    case 3: hipLaunchKernelGGL(mfma_issue_kernel<3>, grid, block, 0, s, d_in, d_out, iters); break;
    default: hipLaunchKernelGGL(mfma_issue_kernel<4>, grid, block, 0, s, d_in, d_out, iters); break;
  }
  return (int)hipGetLastError();
}

// Compute units of the current device (the probe's sink holds 4 per unit
// and workgroup per unit).
extern "C" int pkv_probe_compute_units(void) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) return -1;
  return cus;
}
