// paged_kv_append and pkv_copy_blocks kernels.
//
// A decode step computes only the new token's K and V and stores them in the
// cache [KV Cache 工程学 §15.1]; with paging the store goes to slot t of the
// physical block named by the sequence's table [§15.5].  The host block
// manager turns (sequence, position) into slot = block*16 + t, so the kernel
// is a bit-exact scatter -- or, for an int8 or FP8 cache [§15.7 (3)], a per-row
// quantisation followed by the scatter.  Copy-on-write duplicates a whole shared block
// before a sequence writes into it [KV Cache 与 PagedAttention, first article].
#include "pkv_device.h"
#include "pkv_internal.h"

namespace {

// One workgroup per token.  A thread moves one 16-byte unit of X elements of
// K and of V: the K unit is contiguous in the pool too (one X-element group of
// the K layout), the V unit's elements land 16 slots apart (the V layout is
// [d][16 tokens]).  The token's rows are requested before its slot id is
// known, so the kernel waits for one round trip of memory, not two.
template <typename E>
__global__ __launch_bounds__(256) void append_kernel(E *__restrict__ kpool, E *__restrict__ vpool,
                                                     const E *__restrict__ k_new, const E *__restrict__ v_new,
                                                     const int64_t *__restrict__ slots, int H, int D,
                                                     int num_blocks) {
  constexpr int X = 16 / sizeof(E);
  const int t = blockIdx.x;
  const int cpr = D / X;  // 16-byte units per head row
  const int units = H * cpr;
  const uint4 *krow = reinterpret_cast<const uint4 *>(k_new + (size_t)t * H * D);
  const uint4 *vrow = reinterpret_cast<const uint4 *>(v_new + (size_t)t * H * D);
  const int64_t s = slots[t];
  for (int i = threadIdx.x; i < units; i += blockDim.x) {
    const uint4 kv = krow[i];
    const uint4 vv = vrow[i];
    if (s < 0 || s >= (int64_t)num_blocks * 16) return;  // uniform across the workgroup
    const int64_t blk = s >> 4;
    const int off = (int)(s & 15);
    const int g = i / cpr, c = i - g * cpr;
    *reinterpret_cast<uint4 *>(kpool + ((((size_t)blk * H + g) * cpr + c) * 16 + off) * X) = kv;
    E ve[X];
    __builtin_memcpy(ve, &vv, sizeof vv);
    E *vdst = vpool + (((size_t)blk * H + g) * D + (size_t)c * X) * 16 + off;
#pragma unroll
    for (int e = 0; e < X; ++e) vdst[e * 16] = ve[e];
  }
}

// Bulk appends (a prompt's tokens): workgroup j takes input tokens
// [16j, 16j + 16).  A run is 16 input tokens whose slots fill one block in
// order (the first slot a multiple of 16, each next one more); at most one run
// starts in a workgroup's range, and that workgroup writes it a block at a
// time: the 16 tokens' K units of one row group land in one contiguous
// 16-unit stretch of the tile, and a thread gathers the 16 tokens' elements
// of one (head, d) into that block's V row (contiguous in the [d][16 tokens]
// layout) and stores it whole -- instead of 16 scattered element stores per
// row.  Tokens of the range that belong to no run are stored one by one as in
// append_kernel; tokens of a run that started in the previous range belong to
// that range's workgroup.  The bytes written are the same either way.
template <typename E>
__global__ __launch_bounds__(256) void append_runs_kernel(E *__restrict__ kpool, E *__restrict__ vpool,
                                                          const E *__restrict__ k_new, const E *__restrict__ v_new,
                                                          const int64_t *__restrict__ slots, int T, int H, int D,
                                                          int num_blocks) {
  constexpr int X = 16 / sizeof(E);
  const int cpr = D / X;  // 16-byte units per head row
  const int units = H * cpr;
  const int64_t nslots = (int64_t)num_blocks * 16;
  const int i0 = blockIdx.x * 16;
  const int tid = threadIdx.x;
  __shared__ int64_t s_slot[48];  // input tokens i0 - 16 .. i0 + 31 (-1: none or invalid)
  __shared__ bool s_start[32];    // run starts among input tokens i0 - 16 .. i0 + 15
  if (tid < 48) {
    const int i = i0 - 16 + tid;
    int64_t v = -1;
    if (i >= 0 && i < T) {
      v = slots[i];
      if (v < 0 || v >= nslots) v = -1;
    }
    s_slot[tid] = v;
  }
  __syncthreads();
  if (tid < 32) {
    const int64_t a = s_slot[tid];
    bool run = a >= 0 && (a & 15) == 0;
    for (int k = 1; k < 16 && run; ++k) run = s_slot[tid + k] == a + k;
    s_start[tid] = run;
  }
  __syncthreads();
  int r = -1;  // the run starting in this range, as an index into s_slot
#pragma unroll
  for (int t = 0; t < 16; ++t)
    if (s_start[16 + t]) r = 16 + t;

  if (r >= 0) {
    const int64_t blk = s_slot[r] >> 4;
    const size_t in0 = (size_t)(i0 - 16 + r) * H * D;  // first token's row
    for (int idx = tid; idx < 16 * units; idx += blockDim.x) {
      const int t = idx & 15, hc = idx >> 4;
      const int h = hc / cpr, c = hc - h * cpr;
      const uint4 kv = *reinterpret_cast<const uint4 *>(k_new + in0 + (size_t)t * H * D + (size_t)h * D + c * X);
      *reinterpret_cast<uint4 *>(kpool + ((((size_t)blk * H + h) * cpr + c) * 16 + t) * X) = kv;
    }
    for (int idx = tid; idx < H * D; idx += blockDim.x) {
      E row[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) row[t] = v_new[in0 + (size_t)t * H * D + idx];
      uint4 *dst = reinterpret_cast<uint4 *>(vpool + ((size_t)blk * H * D + idx) * 16);
#pragma unroll
      for (int q = 0; q < 16 * (int)sizeof(E) / 16; ++q) {
        uint4 u;
        __builtin_memcpy(&u, reinterpret_cast<const char *>(row) + 16 * q, 16);
        dst[q] = u;
      }
    }
  }
  // Tokens of the range outside every run, one unit of K and V at a time.
  for (int idx = tid; idx < 16 * units; idx += blockDim.x) {
    const int t = idx / units, i = idx - t * units;
    const int64_t s = s_slot[16 + t];
    if (s < 0) continue;
    const int rs = 16 + t - (int)(s & 15);  // where its run would start
    if (s_start[rs]) continue;
    const size_t in = (size_t)(i0 + t) * H * D;
    const uint4 kv = reinterpret_cast<const uint4 *>(k_new + in)[i];
    const uint4 vv = reinterpret_cast<const uint4 *>(v_new + in)[i];
    const int64_t blk = s >> 4;
    const int off = (int)(s & 15);
    const int g = i / cpr, c = i - g * cpr;
    *reinterpret_cast<uint4 *>(kpool + ((((size_t)blk * H + g) * cpr + c) * 16 + off) * X) = kv;
    E ve[X];
    __builtin_memcpy(ve, &vv, sizeof vv);
    E *vdst = vpool + (((size_t)blk * H + g) * D + (size_t)c * X) * 16 + off;
#pragma unroll
    for (int e = 0; e < X; ++e) vdst[e * 16] = ve[e];
  }
}

// The FP8 E4M3 code (OCP format: bias 7, subnormals m/8 * 2^-6, largest
// finite 448) of the value nearest to y, ties to the even mantissa,
// saturated at 448, sign kept; y is finite.  Below 2^-6 the codes are the
// multiples of 2^-9 (code 8 is 2^-6 itself).  Above it the float32 mantissa
// is rounded to 3 bits in the integer domain, a carry moving into the
// exponent, and the exponent is re-biased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t sign = (b >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t c;
  if (a >= 448.f) {
    c = 0x7Eu;
  } else if (a < 0x1p-6f) {
    c = (uint32_t)rintf(a * 512.f);
  } else {
    const uint32_t m = b & 0x7fffffffu;
    c = ((m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sign | c;
}

// int8 and FP8 caches.  A group of D/8 lanes quantises one (token, kv head)
// row of K and one of V; a lane holds 8 consecutive bf16 elements of each.
// The row's largest magnitude comes from xor-shuffles inside the group, then
// every lane divides its elements by scale = amax / 127 (int8) or amax / 448
// (FP8) in float32 (correctly rounded division) and codes the quotient: int8
// rounds half to even and clamps to [-127, 127]; FP8 takes the nearest E4M3
// value.  Codes go to the tile's K and V layouts and lane 0 of the group
// writes the two scales after the tile's codes.
template <int D, bool F8>
__global__ __launch_bounds__(256) void append_q8_kernel(uint8_t *__restrict__ kpool, uint8_t *__restrict__ vpool,
                                                        const uint16_t *__restrict__ k_new,
                                                        const uint16_t *__restrict__ v_new,
                                                        const int64_t *__restrict__ slots, int64_t rows, int H,
                                                        int num_blocks) {
  constexpr int LPR = D / 8;  // lanes per row
  constexpr int TB = 16 * D + 64;
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  const int64_t r = row < rows ? row : 0;  // surplus groups work on row 0 and store nothing
  const int64_t t = r / H;
  const int g = (int)(r - t * H);
  const uint4 kx = *reinterpret_cast<const uint4 *>(k_new + r * D + 8 * part);
  const uint4 vx = *reinterpret_cast<const uint4 *>(v_new + r * D + 8 * part);
  const int64_t s = slots[t];
  float kf[8], vf[8];
  const uint32_t kw[4] = {kx.x, kx.y, kx.z, kx.w}, vw[4] = {vx.x, vx.y, vx.z, vx.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kf[2 * e] = __uint_as_float(kw[e] << 16);
    kf[2 * e + 1] = __uint_as_float(kw[e] & 0xffff0000u);
    vf[2 * e] = __uint_as_float(vw[e] << 16);
    vf[2 * e + 1] = __uint_as_float(vw[e] & 0xffff0000u);
  }
  float ka = 0.f, va = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    ka = fmaxf(ka, fabsf(kf[e]));
    va = fmaxf(va, fabsf(vf[e]));
  }
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) {
    ka = fmaxf(ka, __shfl_xor(ka, o, LPR));
    va = fmaxf(va, __shfl_xor(va, o, LPR));
  }
  if (row >= rows || s < 0 || s >= (int64_t)num_blocks * 16) return;
  constexpr float kTop = F8 ? 448.0f : 127.0f;
  const float ks = ka / kTop, vs = va / kTop;
  uint32_t kc[2] = {0u, 0u};
  uint8_t vc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t kq, vq;
    if constexpr (F8) {
      kq = ka > 0.f ? e4m3_code(kf[e] / ks) : 0u;
      vq = va > 0.f ? e4m3_code(vf[e] / vs) : 0u;
    } else {
      kq = ka > 0.f ? (uint32_t)(int)fminf(fmaxf(rintf(kf[e] / ks), -127.f), 127.f) : 0u;
      vq = va > 0.f ? (uint32_t)(int)fminf(fmaxf(rintf(vf[e] / vs), -127.f), 127.f) : 0u;
    }
    kc[e >> 2] |= (kq & 0xffu) << (8 * (e & 3));
    vc[e] = (uint8_t)(vq & 0xffu);
  }
  const int64_t blk = s >> 4;
  const int off = (int)(s & 15);
  const int d0 = 8 * part;
  uint8_t *kt = kpool + ((size_t)blk * H + g) * TB;
  uint8_t *vt = vpool + ((size_t)blk * H + g) * TB;
  *reinterpret_cast<uint2 *>(kt + ((d0 >> 4) * 16 + k8_unit(off)) * 16 + (d0 & 15)) = make_uint2(kc[0], kc[1]);
#pragma unroll
  for (int e = 0; e < 8; ++e) vt[(d0 + e) * 16 + off] = vc[e];
  if (part == 0) {
    *reinterpret_cast<float *>(kt + 16 * D + 4 * off) = ks;
    *reinterpret_cast<float *>(vt + 16 * D + 4 * off) = vs;
  }
}

// One workgroup per (pair, pool): a block's tiles for all heads are one
// contiguous run of H tiles in either pool.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4 *__restrict__ kpool, uint4 *__restrict__ vpool,
                                                          const int32_t *__restrict__ pairs, int units_per_block,
                                                          int num_blocks) {
  const int src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint4 *pool = blockIdx.y == 0 ? kpool : vpool;
  const uint4 *from = pool + (size_t)src * units_per_block;
  uint4 *to = pool + (size_t)dst * units_per_block;
  for (int i = threadIdx.x; i < units_per_block; i += blockDim.x) to[i] = from[i];
}

// Blocks between two pools of the same layout (either may be pinned host
// memory, read or written over PCIe): workgroup (pair, pool) moves one block's
// tiles for all heads.  Pairs naming a block outside either pool are skipped.
__global__ __launch_bounds__(256) void swap_blocks_kernel(uint4 *__restrict__ dst_k, uint4 *__restrict__ dst_v,
                                                          const uint4 *__restrict__ src_k,
                                                          const uint4 *__restrict__ src_v,
                                                          const int32_t *__restrict__ pairs, int units_per_block,
                                                          int src_blocks, int dst_blocks) {
  const int src = pairs[2 * blockIdx.x], dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const uint4 *from = (blockIdx.y == 0 ? src_k : src_v) + (size_t)src * units_per_block;
  uint4 *to = (blockIdx.y == 0 ? dst_k : dst_v) + (size_t)dst * units_per_block;
  for (int i = threadIdx.x; i < units_per_block; i += blockDim.x) to[i] = from[i];
}

}  // namespace

int pkv_launch_swap(const pkv_layout *L, void *dst_k, void *dst_v, int32_t dst_blocks, const void *src_k,
                    const void *src_v, int32_t src_blocks, const int32_t *pairs, int32_t num_pairs, void *stream) {
  if (num_pairs == 0) return 0;
  const int units = (int)(L->num_kv_heads * pkv_tile_bytes(L) / 16);
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(num_pairs, 2), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     (uint4 *)dst_k, (uint4 *)dst_v, (const uint4 *)src_k, (const uint4 *)src_v, pairs, units,
                     src_blocks, dst_blocks);
  return (int)hipGetLastError();
}

// Appends of at least this many tokens (prompts) take the block-run kernel;
// a decode step's one token per sequence keeps one workgroup per token.
#ifndef PKV_BULK_APPEND_TOKENS
#define PKV_BULK_APPEND_TOKENS 256
#endif
constexpr int kBulkTokens = PKV_BULK_APPEND_TOKENS;

int pkv_launch_append(const pkv_layout *L, void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                      const int64_t *slots, int32_t num_tokens, void *stream) {
  if (num_tokens == 0) return 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (pkv_is_q8(L->kv_dtype)) {
    const int64_t rows = (int64_t)num_tokens * L->num_kv_heads;
    const int per_block = 256 / (L->head_dim / 8);
    const dim3 grid((unsigned)((rows + per_block - 1) / per_block));
    const bool f8 = L->kv_dtype == PKV_FP8;
    auto kern = L->head_dim == 128 ? (f8 ? append_q8_kernel<128, true> : append_q8_kernel<128, false>)
                                   : (f8 ? append_q8_kernel<64, true> : append_q8_kernel<64, false>);
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, (uint8_t *)k_pool, (uint8_t *)v_pool, (const uint16_t *)k_new,
                       (const uint16_t *)v_new, slots, rows, L->num_kv_heads, L->num_blocks);
    return (int)hipGetLastError();
  }
  if (num_tokens >= kBulkTokens) {
    const dim3 grid((unsigned)((num_tokens + 15) / 16));
    if (L->kv_dtype == PKV_BF16)
      hipLaunchKernelGGL(append_runs_kernel<uint16_t>, grid, dim3(256), 0, st, (uint16_t *)k_pool, (uint16_t *)v_pool,
                         (const uint16_t *)k_new, (const uint16_t *)v_new, slots, num_tokens, L->num_kv_heads,
                         L->head_dim, L->num_blocks);
    else
      hipLaunchKernelGGL(append_runs_kernel<float>, grid, dim3(256), 0, st, (float *)k_pool, (float *)v_pool,
                         (const float *)k_new, (const float *)v_new, slots, num_tokens, L->num_kv_heads,
                         L->head_dim, L->num_blocks);
    return (int)hipGetLastError();
  }
  const int units = L->num_kv_heads * L->head_dim * pkv_elem_bytes(L->kv_dtype) / 16;
  dim3 grid(num_tokens), block(units < 256 ? (units + 63) / 64 * 64 : 256);
  if (L->kv_dtype == PKV_BF16)
    hipLaunchKernelGGL(append_kernel<uint16_t>, grid, block, 0, st, (uint16_t *)k_pool, (uint16_t *)v_pool,
                       (const uint16_t *)k_new, (const uint16_t *)v_new, slots, L->num_kv_heads, L->head_dim,
                       L->num_blocks);
  else
    hipLaunchKernelGGL(append_kernel<float>, grid, block, 0, st, (float *)k_pool, (float *)v_pool,
                       (const float *)k_new, (const float *)v_new, slots, L->num_kv_heads, L->head_dim,
                       L->num_blocks);
  return (int)hipGetLastError();
}

int pkv_launch_copy_blocks(const pkv_layout *L, void *k_pool, void *v_pool, const int32_t *pairs,
                           int32_t num_pairs, void *stream) {
  if (num_pairs == 0) return 0;
  const int units = (int)(L->num_kv_heads * pkv_tile_bytes(L) / 16);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     (uint4 *)k_pool, (uint4 *)v_pool, pairs, units, L->num_blocks);
  return (int)hipGetLastError();
}
