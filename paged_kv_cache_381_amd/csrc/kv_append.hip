// paged_kv_append and pkv_copy_blocks kernels.
//
// A decode step computes only the new token's K and V and stores them in the
// cache [KV Cache 工程学 §15.1]; with paging the store goes to slot t of the
// physical block named by the sequence's table [§15.5].  The host block
// manager turns (sequence, position) into slot = block*16 + t, so the kernel
// is a bit-exact scatter.  Copy-on-write duplicates a whole shared block
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

// One workgroup per (pair, pool): a block's tiles for all heads are one
// contiguous run of H*16*D elements in either pool.
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

}  // namespace

int pkv_launch_append(const pkv_layout *L, void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                      const int64_t *slots, int32_t num_tokens, void *stream) {
  if (num_tokens == 0) return 0;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
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
  const int units = L->num_kv_heads * 16 * L->head_dim * pkv_elem_bytes(L->kv_dtype) / 16;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     (uint4 *)k_pool, (uint4 *)v_pool, pairs, units, L->num_blocks);
  return (int)hipGetLastError();
}
