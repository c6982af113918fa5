// C-ABI entry points of the device path: argument validation, workspace
// sizing and kernel dispatch.  See include/pagedkv.h for the contract.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pagedkv.h"
#include "pkv_internal.h"

namespace {

int hip_fail(int rc, const char *what) {
  return pkv_set_error(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(static_cast<hipError_t>(rc)));
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int record(void *ev, void *stream) {
  if (!ev) return PKV_OK;
  hipError_t e = hipEventRecord(reinterpret_cast<hipEvent_t>(ev), reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_fail((int)e, "hipEventRecord");
}

int partition_tokens(const pkv_decode_opts *opts, int32_t *out) {
  int32_t p = (opts && opts->partition_tokens > 0) ? opts->partition_tokens : PKV_DEFAULT_PARTITION;
  if (opts && opts->partition_tokens < 0) return pkv_set_error(PKV_ERR_INVALID, "partition_tokens < 0");
  if (p % PKV_PARTITION_QUANTUM != 0 || p > (1 << 24))
    return pkv_set_error(PKV_ERR_INVALID, "partition_tokens must be a positive multiple of %d (got %d)",
                         PKV_PARTITION_QUANTUM, p);
  *out = p;
  return PKV_OK;
}

int32_t num_partitions(int32_t max_ctx, int32_t part) {
  int32_t np = (max_ctx + part - 1) / part;
  return np < 1 ? 1 : np;
}

}  // namespace

extern "C" int paged_kv_append(const pkv_layout *layout, void *k_pool, void *v_pool, const void *k_new,
                               const void *v_new, const int64_t *d_slots, int32_t num_tokens, void *stream) {
  if (int rc = pkv_check_layout(layout)) return rc;
  if (num_tokens < 0) return pkv_set_error(PKV_ERR_INVALID, "num_tokens < 0");
  if (num_tokens == 0) return PKV_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !d_slots)
    return pkv_set_error(PKV_ERR_INVALID, "paged_kv_append: NULL pointer");
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) ||
      !aligned(d_slots, 8))
    return pkv_set_error(PKV_ERR_INVALID, "paged_kv_append: pools and token rows must be 16-byte aligned");
  if (int rc = pkv_launch_append(layout, k_pool, v_pool, k_new, v_new, d_slots, num_tokens, stream))
    return hip_fail(rc, "paged_kv_append launch");
  return PKV_OK;
}

extern "C" int pkv_copy_blocks(const pkv_layout *layout, void *k_pool, void *v_pool, const int32_t *d_pairs,
                               int32_t num_pairs, void *stream) {
  if (int rc = pkv_check_layout(layout)) return rc;
  if (num_pairs < 0) return pkv_set_error(PKV_ERR_INVALID, "num_pairs < 0");
  if (num_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !d_pairs) return pkv_set_error(PKV_ERR_INVALID, "pkv_copy_blocks: NULL pointer");
  if (!aligned(k_pool, 16) || !aligned(v_pool, 16))
    return pkv_set_error(PKV_ERR_INVALID, "pkv_copy_blocks: pools must be 16-byte aligned");
  if (num_pairs > 65535 * 32767) return pkv_set_error(PKV_ERR_INVALID, "too many pairs");
  if (int rc = pkv_launch_copy_blocks(layout, k_pool, v_pool, d_pairs, num_pairs, stream))
    return hip_fail(rc, "pkv_copy_blocks launch");
  return PKV_OK;
}

extern "C" size_t paged_attention_workspace_bytes(const pkv_layout *layout, int32_t num_seqs, int32_t num_q_heads,
                                                  int32_t max_context_len, const pkv_decode_opts *opts) {
  if (pkv_check_layout(layout) || num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0) return 0;
  int32_t part;
  if (partition_tokens(opts, &part)) return 0;
  const int32_t np = num_partitions(max_context_len, part);
  if (np <= 1) return 0;
  return (size_t)num_seqs * num_q_heads * np * (layout->head_dim + 2) * sizeof(float);
}

extern "C" int paged_attention_decode(const pkv_layout *layout, float *out, const void *q, const void *k_pool,
                                      const void *v_pool, const int32_t *d_block_tables,
                                      const int32_t *d_context_lens, int32_t num_seqs, int32_t num_q_heads,
                                      int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                      void *workspace, size_t workspace_bytes, const pkv_decode_opts *opts,
                                      void *stream) {
  if (int rc = pkv_check_layout(layout)) return rc;
  const int32_t H = layout->num_kv_heads;
  if (num_seqs < 0) return pkv_set_error(PKV_ERR_INVALID, "num_seqs < 0");
  if (num_q_heads <= 0 || num_q_heads % H != 0)
    return pkv_set_error(PKV_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                         num_q_heads, H);
  const int32_t G = num_q_heads / H;
  if (G > 16) return pkv_set_error(PKV_ERR_INVALID, "query heads per kv head must be <= 16 (got %d)", G);
  if (max_blocks_per_seq <= 0) return pkv_set_error(PKV_ERR_INVALID, "max_blocks_per_seq must be > 0");
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)PKV_BLOCK_SIZE * max_blocks_per_seq)
    return pkv_set_error(PKV_ERR_INVALID, "max_context_len %d outside [0, 16 * max_blocks_per_seq]",
                         max_context_len);
  if (!std::isfinite(scale)) return pkv_set_error(PKV_ERR_INVALID, "scale is not finite");
  if (num_seqs > 65535 || H > 65535) return pkv_set_error(PKV_ERR_INVALID, "grid too large");
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !d_block_tables || !d_context_lens)
    return pkv_set_error(PKV_ERR_INVALID, "paged_attention_decode: NULL pointer");
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 4))
    return pkv_set_error(PKV_ERR_INVALID, "paged_attention_decode: q and pools must be 16-byte aligned");
  int32_t part;
  if (int rc = partition_tokens(opts, &part)) return rc;
  int kernel = opts ? opts->kernel : 0;
  if (kernel == 0) kernel = (layout->kv_dtype == PKV_BF16 && G >= 4) ? 2 : 1;
  if (kernel != 1 && kernel != 2) return pkv_set_error(PKV_ERR_INVALID, "unknown kernel %d", kernel);
  if (kernel == 2 && layout->kv_dtype != PKV_BF16)
    return pkv_set_error(PKV_ERR_INVALID, "the matrix-core kernel needs a bf16 cache");

  const int32_t np = num_partitions(max_context_len, part);
  const size_t need = paged_attention_workspace_bytes(layout, num_seqs, num_q_heads, max_context_len, opts);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 4)))
    return pkv_set_error(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                         workspace ? workspace_bytes : (size_t)0);

  pkv_decode_args a{};
  a.L = layout;
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.tables = d_block_tables;
  a.ctx = d_context_lens;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.max_blocks = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.part_tokens = part;
  a.num_parts = np;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.ws_o = need ? static_cast<float *>(workspace) : nullptr;
  a.ws_ml = need ? static_cast<float *>(workspace) + (size_t)num_seqs * num_q_heads * np * layout->head_dim : nullptr;
  a.stream = stream;

  if (int rc = record(opts ? opts->ev_begin : nullptr, stream)) return rc;
  const int rc = kernel == 2 ? pkv_launch_decode_mfma(a) : pkv_launch_decode_valu(a);
  if (rc) return hip_fail(rc, "decode partition kernel launch");
  if (int r = record(opts ? opts->ev_partition_done : nullptr, stream)) return r;
  if (np > 1) {
    if (int r2 = pkv_launch_merge(a)) return hip_fail(r2, "merge kernel launch");
  }
  return record(opts ? opts->ev_end : nullptr, stream);
}
