// Internal declarations shared by the library's translation units.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

// Record a thread-local error message and return code.
int pkv_set_error(int code, const char *fmt, ...);
// Validate a pkv_layout; PKV_OK or PKV_ERR_INVALID with a message.
int pkv_check_layout(const pkv_layout *L);

// Bytes of one stored element (a one-byte code for PKV_INT8 and PKV_FP8).
inline int pkv_elem_bytes(int dtype) { return dtype == PKV_F32 ? 4 : dtype == PKV_BF16 ? 2 : 1; }
// One-byte codes with a float32 scale per (token, kv head) row.
inline bool pkv_is_q8(int dtype) { return dtype == PKV_INT8 || dtype == PKV_FP8; }
// Bytes of one (block, kv head) tile of a pool: 16 token slots of D elements,
// plus the 16 float32 scales of an int8 or FP8 tile.
inline int64_t pkv_tile_bytes(const pkv_layout *L) {
  return (int64_t)PKV_BLOCK_SIZE * L->head_dim * pkv_elem_bytes(L->kv_dtype) +
         (pkv_is_q8(L->kv_dtype) ? 4 * PKV_BLOCK_SIZE : 0);
}
// Bytes of one token's K (or V) row of one kv head, its scale included.
inline int64_t pkv_row_bytes(const pkv_layout *L) {
  return (int64_t)L->head_dim * pkv_elem_bytes(L->kv_dtype) + (pkv_is_q8(L->kv_dtype) ? 4 : 0);
}


// XCDs of the chip: regions of the chunk list that can be weighted.
#define PKV_REGIONS 8
// Schedule header ints ahead of the chunk scan: chunks per kv head, waves
// used, regions, a pad, then PKV_REGIONS + 1 int64 region bounds.
#define PKV_HDR_INTS (4 + 2 * (PKV_REGIONS + 1))
// Ints a decode wave writes to a trace buffer (PKV_TRACE_WAVES waves).
#define PKV_TRACE_INTS 4
// Ints of one wave's record in a decode plan, and the chunks whose cursor
// and blocks a record holds.
#define PKV_PLAN_REC_INTS 32
#define PKV_PLAN_CHUNKS 2
// Ints of a plan's clamped lengths, padded so that the records after them
// start 16-byte aligned.
constexpr int pkv_plan_lens_ints(int num_seqs) { return (num_seqs + 3) & ~3; }
// Most waves a decode grid runs: 8 per compute unit of MI355X's 256 (one or
// two workgroups of four waves).  Bounds the partial slots of the workspace.
#define PKV_MAX_DECODE_WAVES 2048

// Kernel launchers (decode_*.hip, kv_append.hip).  They return a HIP error
// code (0 = success); arguments were validated by the caller.
struct pkv_decode_args {
  const pkv_layout *L;
  float *out;
  const void *q;
  const void *k_pool;
  const void *v_pool;
  const int32_t *tables;
  const int32_t *ctx;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t max_blocks;
  int32_t max_ctx;
  float scale_log2;  // scale * log2(e): scores are kept in base 2
  float *ws_o;       // [nslots][G][D] partial outputs
  float *ws_ml;      // [nslots][G][2] partial (max, sum)
  int32_t *ws_hdr;   // [PKV_HDR_INTS + B] schedule header of the merge kernel
  int32_t xw[PKV_REGIONS];  // per-XCD weights of the work (all 0: equal shares)
  int32_t *trace;    // nullable device buffer: PKV_TRACE_INTS per wave
  int32_t nslots;    // partial slots: two per wave (its first and its last segment)
  int32_t min_cpw;   // fewest 32-token chunks per wave
  int32_t kernel;          // 1 wavefront reductions, 2 matrix cores
  int32_t waves_per_simd;  // resident waves per SIMD of the matrix-core kernel (1 or 2)
  int32_t streaming;       // K/V tiles read with non-temporal loads (1) or cached ones (0)
  int32_t plan_mode;       // matrix-core kernel: 0 schedules itself, 1 runs from a plan, 2 writes one
  int32_t *plan;           // plan region of the workspace (plan_mode 1 and 2)
  int32_t plan_cap;        // records of the plan region
  void *stream;
};

// Tokens per chunk of the balanced-split kernels.
#define PKV_CHUNK 32
// Default fewest chunks given to one wave by the balanced split.
#ifndef PKV_DEFAULT_MIN_CHUNKS
#define PKV_DEFAULT_MIN_CHUNKS 4
#endif
// Dynamic LDS that keeps a CU (160 KiB of LDS) to one workgroup.
#define PKV_LDS_ONE_WG_PER_CU (81 * 1024)
// Largest batch of the balanced split (its chunk scan lives in LDS).
#define PKV_MAX_SPLIT_SEQS 8192

// Persistent grid of a balanced-split kernel: workgroups resident at once on
// the device (occupancy x compute units), capped by the work, a multiple of 8.
int pkv_split_grid(const void *kernel, int block_threads, size_t lds_bytes, const pkv_decode_args &a, int *nwg);

int pkv_launch_append(const pkv_layout *L, void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                      const int64_t *slots, int32_t num_tokens, void *stream);
int pkv_launch_swap(const pkv_layout *L, void *dst_k, void *dst_v, int32_t dst_blocks, const void *src_k,
                    const void *src_v, int32_t src_blocks, const int32_t *pairs, int32_t num_pairs, void *stream);
int pkv_launch_copy_blocks(const pkv_layout *L, void *k_pool, void *v_pool, const int32_t *pairs,
                           int32_t num_pairs, void *stream);
struct pkv_prefill_args {
  const pkv_layout *L;
  float *out;
  const void *q;
  const void *k_pool;
  const void *v_pool;
  const int32_t *tables;
  const int32_t *ctx;
  const int32_t *qstart;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t max_blocks;
  int32_t max_ctx;
  int32_t max_query_len;
  float scale_log2;
  void *stream;
};
int pkv_launch_prefill_mfma(const pkv_prefill_args &a);
int pkv_launch_decode_valu(const pkv_decode_args &a);
int pkv_launch_decode_mfma(const pkv_decode_args &a);
int pkv_launch_merge(const pkv_decode_args &a);
