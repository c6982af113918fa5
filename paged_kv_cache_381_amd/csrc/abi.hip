// C-ABI entry points of the device path: argument validation, workspace
// sizing and kernel dispatch.  See include/pagedkv.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

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

// Fewest chunks per wave of the balanced split, from opts->partition_tokens
// (fewest tokens per wave: a positive multiple of 32, or 0 for the default).
int min_chunks(const pkv_decode_opts *opts, int32_t *out) {
  const int32_t p = opts ? opts->partition_tokens : 0;
  if (p < 0 || p % PKV_CHUNK != 0 || p > (1 << 22))
    return pkv_set_error(PKV_ERR_INVALID, "partition_tokens must be 0 or a positive multiple of %d up to %d (got %d)",
                         PKV_CHUNK, 1 << 22, p);
  *out = p > 0 ? p / PKV_CHUNK : PKV_DEFAULT_MIN_CHUNKS;
  return PKV_OK;
}

// Kernel a call runs: 1 wavefront reductions, 2 matrix cores (int8 and FP8,
// and bf16 with G >= 4, by default).
int choose_kernel(const pkv_layout *L, int32_t G, const pkv_decode_opts *opts) {
  const int k = opts ? opts->kernel : 0;
  if (k != 0) return k;
  if (pkv_is_q8(L->kv_dtype)) return 2;
  return (L->kv_dtype == PKV_BF16 && G >= 4) ? 2 : 1;
}

size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Partial slots of the balanced split: two per wave that can receive work
// (only its first and its last segment can be cut), and a grid has at most
// PKV_MAX_DECODE_WAVES waves and never more working waves than chunks over
// min_cpw.
int32_t split_slots(int32_t B, int32_t H, int32_t max_ctx, int32_t min_cpw) {
  const int64_t chunks = (int64_t)B * H * ((max_ctx + PKV_CHUNK - 1) / PKV_CHUNK);
  const int64_t waves = std::max<int64_t>(1, std::min<int64_t>(PKV_MAX_DECODE_WAVES, chunks / min_cpw));
  return (int32_t)(2 * waves);
}

// Workspace of the balanced split: partial outputs [nslots][G][D] and
// (m, l) [nslots][G] of float32, then the merge kernel's schedule header
// (PKV_HDR_INTS + B int32), each region padded to 16 bytes.
size_t split_ws_bytes(const pkv_layout *L, int32_t B, int32_t Hq, int32_t nslots) {
  const size_t rows = (size_t)nslots * (Hq / L->num_kv_heads);
  return align16(rows * L->head_dim * sizeof(float)) + align16(rows * 2 * sizeof(float)) +
         align16((size_t)(PKV_HDR_INTS + B) * sizeof(int32_t));
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
  if ((int64_t)num_tokens * layout->num_kv_heads > ((int64_t)1 << 34))
    return pkv_set_error(PKV_ERR_INVALID, "paged_kv_append: too many rows");
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

int pkv_split_grid(const void *kernel, int block_threads, size_t lds_bytes, const pkv_decode_args &a, int *nwg) {
  struct Occ {
    const void *kernel;
    int device;
    size_t lds;
    int per_cu;
    int cus;
  };
  static thread_local Occ cache[16] = {};
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return (int)e;
  Occ *hit = nullptr;
  for (Occ &c : cache)
    if (c.kernel == kernel && c.device == dev && c.lds == lds_bytes) hit = &c;
  if (!hit) {
    Occ o{kernel, dev, lds_bytes, 0, 0};
    if (lds_bytes > 65536) {
      if (hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes))
        return (int)e;
    }
    if (hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&o.per_cu, kernel, block_threads, lds_bytes))
      return (int)e;
    if (hipError_t e = hipDeviceGetAttribute(&o.cus, hipDeviceAttributeMultiprocessorCount, dev)) return (int)e;
    for (int i = 15; i > 0; --i) cache[i] = cache[i - 1];
    cache[0] = o;
    hit = &cache[0];
  }
  const int waves_per_wg = block_threads / 64;
  int64_t grid = (int64_t)std::max(1, hit->per_cu) * std::max(1, hit->cus);
  // The workspace holds partial slots for at most PKV_MAX_DECODE_WAVES waves.
  static_assert(PKV_MAX_DECODE_WAVES % (8 * 4) == 0, "the wave cap must stay a multiple of 8 workgroups");
  grid = std::min<int64_t>(grid, PKV_MAX_DECODE_WAVES / waves_per_wg);
  // No more workgroups than the largest possible batch of chunks can feed.
  const int64_t max_chunks = (int64_t)a.num_seqs * a.L->num_kv_heads * ((a.max_ctx + PKV_CHUNK - 1) / PKV_CHUNK);
  const int64_t need = (max_chunks + (int64_t)a.min_cpw * waves_per_wg - 1) / ((int64_t)a.min_cpw * waves_per_wg);
  grid = std::min(grid, std::max<int64_t>(need, 1));
  *nwg = (int)((grid + 7) & ~(int64_t)7);
  return 0;
}


extern "C" size_t paged_attention_workspace_bytes(const pkv_layout *layout, int32_t num_seqs, int32_t num_q_heads,
                                                  int32_t max_context_len, const pkv_decode_opts *opts) {
  if (pkv_check_layout(layout) || num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0) return 0;
  if (num_q_heads % layout->num_kv_heads) return 0;
  int32_t mc;
  if (min_chunks(opts, &mc)) return 0;
  return split_ws_bytes(layout, num_seqs, num_q_heads, split_slots(num_seqs, layout->num_kv_heads, max_context_len, mc));
}

namespace {

// Validation shared by the decode entry points and the arguments of the
// launch, all but the workspace regions.  Returns PKV_OK, an error, or 1 when
// the call has nothing to do (no sequences).
int decode_prepare(const pkv_layout *layout, float *out, const void *q, const void *k_pool, const void *v_pool,
                   const int32_t *d_block_tables, const int32_t *d_context_lens, int32_t num_seqs,
                   int32_t num_q_heads, int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                   const pkv_decode_opts *opts, void *stream, pkv_decode_args *a) {
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
  if (num_seqs == 0) return 1;
  if (!out || !q || !k_pool || !v_pool || !d_block_tables || !d_context_lens)
    return pkv_set_error(PKV_ERR_INVALID, "paged_attention_decode: NULL pointer");
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 4))
    return pkv_set_error(PKV_ERR_INVALID, "paged_attention_decode: q and pools must be 16-byte aligned");
  int32_t mc;
  if (int rc = min_chunks(opts, &mc)) return rc;
  const int kernel = choose_kernel(layout, G, opts);
  if (kernel != 1 && kernel != 2) return pkv_set_error(PKV_ERR_INVALID, "unknown kernel %d", kernel);
  if (opts && (opts->waves_per_simd < 0 || opts->waves_per_simd > 2))
    return pkv_set_error(PKV_ERR_INVALID, "waves_per_simd must be 0, 1 or 2 (got %d)", opts->waves_per_simd);
  if (opts && (opts->load_policy < 0 || opts->load_policy > 2))
    return pkv_set_error(PKV_ERR_INVALID, "load_policy must be 0, 1 or 2 (got %d)", opts->load_policy);
  if (kernel == 2 && layout->kv_dtype == PKV_F32)
    return pkv_set_error(PKV_ERR_INVALID, "the matrix-core kernel needs a bf16, int8 or FP8 cache");
  if (kernel == 1 && pkv_is_q8(layout->kv_dtype))
    return pkv_set_error(PKV_ERR_INVALID, "an int8 or FP8 cache is read by the matrix-core kernel only");
  if (opts)
    for (int i = 0; i < PKV_REGIONS; ++i)
      if (opts->xcd_weights[i] < 0 || opts->xcd_weights[i] > (1 << 20))
        return pkv_set_error(PKV_ERR_INVALID, "xcd_weights[%d] = %d outside [0, 2^20]", i, opts->xcd_weights[i]);
  if (num_seqs > PKV_MAX_SPLIT_SEQS)
    return pkv_set_error(PKV_ERR_INVALID, "at most %d sequences per call (got %d)", PKV_MAX_SPLIT_SEQS, num_seqs);
  if (max_context_len > (1 << 22))
    return pkv_set_error(PKV_ERR_INVALID, "max_context_len %d exceeds %d", max_context_len, 1 << 22);

  a->L = layout;
  a->out = out;
  a->q = q;
  a->k_pool = k_pool;
  a->v_pool = v_pool;
  a->tables = d_block_tables;
  a->ctx = d_context_lens;
  a->num_seqs = num_seqs;
  a->num_q_heads = num_q_heads;
  a->max_blocks = max_blocks_per_seq;
  a->max_ctx = max_context_len;
  a->scale_log2 = scale * 1.4426950408889634f;
  a->stream = stream;
  a->min_cpw = mc;
  a->kernel = kernel;
  a->waves_per_simd = opts && opts->waves_per_simd ? opts->waves_per_simd : 1;
  const int policy = opts ? opts->load_policy : 0;
  // Auto: streaming loads for bf16 and f32 caches read by one wave per SIMD
  // (measured: 8B-shaped batch 104.8 -> 95.7 us, 70B-shaped 732 -> 660 us);
  // cached loads for one-byte caches (streaming measured 9 % slower there)
  // and for batches of mostly shared blocks (two waves per SIMD), which L2
  // serves.
  a->streaming = policy == 1 || (policy == 0 && a->waves_per_simd == 1 && !pkv_is_q8(layout->kv_dtype));
  a->nslots = split_slots(num_seqs, H, max_context_len, mc);
  for (int i = 0; i < PKV_REGIONS; ++i) a->xw[i] = opts ? opts->xcd_weights[i] : 0;
  a->trace = opts ? opts->trace : nullptr;
  return PKV_OK;
}

// The workspace regions of a prepared call: partial outputs, partial
// (m, l), schedule header (the layout of paged_attention_workspace_bytes).
void carve_workspace(pkv_decode_args *a, void *workspace) {
  const size_t rows = (size_t)a->nslots * (a->num_q_heads / a->L->num_kv_heads);
  char *ws = static_cast<char *>(workspace);
  a->ws_o = reinterpret_cast<float *>(ws);
  a->ws_ml = reinterpret_cast<float *>(ws + align16(rows * a->L->head_dim * sizeof(float)));
  a->ws_hdr = reinterpret_cast<int32_t *>(ws + align16(rows * a->L->head_dim * sizeof(float)) +
                                          align16(rows * 2 * sizeof(float)));
}

// ------------------------------------------------------------ decode plans
// A plan buffer holds the schedule header the merge kernel reads (as in a
// workspace, padded to 16 bytes), then the clamped lengths (padded to 4
// ints) and one record of PKV_PLAN_REC_INTS per wave that can receive work.
int32_t plan_cap(const pkv_decode_args &a) { return a.nslots / 2; }
size_t plan_hdr_bytes(int32_t B) { return align16((size_t)(PKV_HDR_INTS + B) * sizeof(int32_t)); }
size_t plan_bytes_of(const pkv_decode_args &a) {
  return plan_hdr_bytes(a.num_seqs) +
         ((size_t)pkv_plan_lens_ints(a.num_seqs) + (size_t)plan_cap(a) * PKV_PLAN_REC_INTS) * sizeof(int32_t);
}

// What a plan was made for: every argument and option that decides the
// schedule or the blocks it names, the plan buffer and the device.
constexpr int64_t kPlanMagic = 0x504b56504c414e31;  // "PKVPLAN1"
int plan_key(const pkv_decode_args &a, const void *d_plan, int64_t key[PKV_PLAN_KEY_INTS]) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return hip_fail((int)e, "hipGetDevice");
  int64_t v[] = {kPlanMagic,
                 dev,
                 (int64_t)reinterpret_cast<uintptr_t>(d_plan),
                 (int64_t)reinterpret_cast<uintptr_t>(a.tables),
                 (int64_t)reinterpret_cast<uintptr_t>(a.ctx),
                 a.num_seqs,
                 a.num_q_heads,
                 a.max_blocks,
                 a.max_ctx,
                 a.L->num_blocks,
                 a.L->num_kv_heads,
                 a.L->head_dim,
                 a.L->kv_dtype,
                 a.kernel,
                 a.min_cpw,
                 a.waves_per_simd,
                 a.streaming,
                 a.xw[0], a.xw[1], a.xw[2], a.xw[3], a.xw[4], a.xw[5], a.xw[6], a.xw[7]};
  static_assert(sizeof(v) / sizeof(v[0]) < PKV_PLAN_KEY_INTS, "the plan key outgrew pkv_decode_plan");
  for (int i = 0; i < PKV_PLAN_KEY_INTS; ++i) key[i] = i < (int)(sizeof(v) / sizeof(v[0])) ? v[i] : 0;
  return PKV_OK;
}

// Which recording each plan buffer holds (the latest one made into it), so
// that a plan whose buffer has been recorded into again since is refused:
// its records would describe another call.  A buffer forgotten here (more
// than kPlanBuffers in use) refuses its plans too, which stays safe.
constexpr int kPlanBuffers = 256;
struct PlanBufferSlot {
  const void *buffer = nullptr;
  int64_t recording = 0;
};
std::mutex g_plan_mu;
PlanBufferSlot g_plan_buffers[kPlanBuffers];
int64_t g_plan_recordings = 0;
int g_plan_next = 0;

int64_t plan_buffer_recorded(const void *buffer) {
  std::lock_guard<std::mutex> lock(g_plan_mu);
  const int64_t id = ++g_plan_recordings;
  for (PlanBufferSlot &b : g_plan_buffers)
    if (b.buffer == buffer) {
      b.recording = id;
      return id;
    }
  g_plan_buffers[g_plan_next] = PlanBufferSlot{buffer, id};
  g_plan_next = (g_plan_next + 1) % kPlanBuffers;
  return id;
}

bool plan_buffer_holds(const void *buffer, int64_t recording) {
  std::lock_guard<std::mutex> lock(g_plan_mu);
  for (const PlanBufferSlot &b : g_plan_buffers)
    if (b.buffer == buffer) return b.recording == recording;
  return false;
}

// Key slot of the recording's number (after the call's description).
constexpr int kPlanRecordingSlot = PKV_PLAN_KEY_INTS - 1;

// A prepared call's use of opts->plan: none, record a fresh plan (an empty
// *opts->plan: the call schedules itself and writes its split to the plan
// buffer), or run from a recorded one after checking that the call is the
// one it was recorded for.  *key receives what the call is.
enum PlanUse { kNoPlan, kRecord, kRun };
int use_plan(pkv_decode_args *a, const pkv_decode_opts *opts, PlanUse *use, int64_t key[PKV_PLAN_KEY_INTS]) {
  *use = kNoPlan;
  if (!opts || !opts->plan) return PKV_OK;
  const size_t need = plan_bytes_of(*a);
  if (!opts->plan_buffer || opts->plan_bytes < need || !aligned(opts->plan_buffer, 16))
    return pkv_set_error(PKV_ERR_WORKSPACE, "a plan buffer of %zu bytes, 16-byte aligned, is needed (got %zu)", need,
                         opts->plan_buffer ? opts->plan_bytes : (size_t)0);
  if (int rc = plan_key(*a, opts->plan_buffer, key)) return rc;
  const int64_t *made = opts->plan->opaque;
  if (made[0] == 0) {
    *use = kRecord;
  } else {
    if (made[0] != kPlanMagic) return pkv_set_error(PKV_ERR_INVALID, "opts->plan holds neither a plan nor zeros");
    for (int i = 0; i < kPlanRecordingSlot; ++i)
      if (key[i] != made[i])
        return pkv_set_error(PKV_ERR_INVALID,
                             "opts->plan was recorded for other arguments, options or device (field %d differs)", i);
    if (!plan_buffer_holds(opts->plan_buffer, made[kPlanRecordingSlot]))
      return pkv_set_error(PKV_ERR_INVALID, "opts->plan: its plan buffer has been recorded into again since");
    *use = kRun;
  }
  if (a->kernel != 2) return PKV_OK;  // the wavefront-reduction kernel schedules itself every call
  a->plan_mode = *use == kRecord ? 2 : 1;
  a->ws_hdr = static_cast<int32_t *>(opts->plan_buffer);
  a->plan = reinterpret_cast<int32_t *>(static_cast<char *>(opts->plan_buffer) + plan_hdr_bytes(a->num_seqs));
  a->plan_cap = plan_cap(*a);
  return PKV_OK;
}

// The partition and merge kernels of a prepared call, between the optional
// events.
int decode_launch(pkv_decode_args &a, const pkv_decode_opts *opts, void *stream) {
  PlanUse use;
  int64_t key[PKV_PLAN_KEY_INTS];
  if (int rc = use_plan(&a, opts, &use, key)) return rc;
  if (int rc = record(opts ? opts->ev_begin : nullptr, stream)) return rc;
  const int rc = a.kernel == 2 ? pkv_launch_decode_mfma(a) : pkv_launch_decode_valu(a);
  if (rc) return hip_fail(rc, "decode partition kernel launch");
  if (int r = record(opts ? opts->ev_partition_done : nullptr, stream)) return r;
  if (int r2 = pkv_launch_merge(a)) return hip_fail(r2, "merge kernel launch");
  if (use == kRecord) {
    key[kPlanRecordingSlot] = plan_buffer_recorded(opts->plan_buffer);
    for (int i = 0; i < PKV_PLAN_KEY_INTS; ++i) opts->plan->opaque[i] = key[i];
  }
  return record(opts ? opts->ev_end : nullptr, stream);
}

}  // namespace

extern "C" int paged_attention_decode(const pkv_layout *layout, float *out, const void *q, const void *k_pool,
                                      const void *v_pool, const int32_t *d_block_tables,
                                      const int32_t *d_context_lens, int32_t num_seqs, int32_t num_q_heads,
                                      int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                      void *workspace, size_t workspace_bytes, const pkv_decode_opts *opts,
                                      void *stream) {
  pkv_decode_args a{};
  const int prep = decode_prepare(layout, out, q, k_pool, v_pool, d_block_tables, d_context_lens, num_seqs,
                                  num_q_heads, max_blocks_per_seq, max_context_len, scale, opts, stream, &a);
  if (prep) return prep == 1 ? PKV_OK : prep;
  const size_t need = paged_attention_workspace_bytes(layout, num_seqs, num_q_heads, max_context_len, opts);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16))
    return pkv_set_error(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need,
                         workspace ? workspace_bytes : (size_t)0);
  carve_workspace(&a, workspace);
  return decode_launch(a, opts, stream);
}

extern "C" size_t paged_attention_plan_bytes(const pkv_layout *layout, int32_t num_seqs, int32_t num_q_heads,
                                             int32_t max_context_len, const pkv_decode_opts *opts) {
  if (pkv_check_layout(layout) || num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0) return 0;
  if (num_q_heads % layout->num_kv_heads) return 0;
  int32_t mc;
  if (min_chunks(opts, &mc)) return 0;
  pkv_decode_args a{};
  a.num_seqs = num_seqs;
  a.nslots = split_slots(num_seqs, layout->num_kv_heads, max_context_len, mc);
  return plan_bytes_of(a);
}

// ------------------------------------------------ decode without allocation
namespace {

// Scratch of paged_attention_decode_noalloc: the workspace of the largest
// call (2 * PKV_MAX_DECODE_WAVES slots of 16 query rows of 128 floats, their
// (m, l), the schedule header of PKV_MAX_SPLIT_SEQS sequences), 32.6 MiB,
// one copy per GPU that the library runs on, held until the process ends.
// Host code never uses this name as an address: it takes the device
// address of each GPU's copy with hipGetSymbolAddress.
constexpr size_t kNoallocRows = (size_t)2 * PKV_MAX_DECODE_WAVES * 16;
constexpr size_t kNoallocBytes = ((kNoallocRows * 128 * sizeof(float) + 15) & ~(size_t)15) +
                                 ((kNoallocRows * 2 * sizeof(float) + 15) & ~(size_t)15) +
                                 (((size_t)(PKV_HDR_INTS + PKV_MAX_SPLIT_SEQS) * sizeof(int32_t) + 15) & ~(size_t)15);
static_assert(kNoallocBytes == 34111584, "the size stated in pagedkv.h");
__device__ __align__(256) uint8_t scratch[kNoallocBytes];

constexpr int kMaxDevices = 64;
struct NoallocScratch {
  std::once_flag once;
  void *ptr = nullptr;
  int rc = 0;
};
NoallocScratch g_noalloc[kMaxDevices];

// The device address of the current GPU's scratch, looked up once per
// device (with that device current) and kept.
int noalloc_scratch(void **out) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return hip_fail((int)e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return pkv_set_error(PKV_ERR_INVALID, "device %d beyond %d", dev, kMaxDevices);
  NoallocScratch &ns = g_noalloc[dev];
  std::call_once(ns.once, [&ns] { ns.rc = (int)hipGetSymbolAddress(&ns.ptr, HIP_SYMBOL(scratch)); });
  if (ns.rc) return hip_fail(ns.rc, "hipGetSymbolAddress of the decode scratch");
  *out = ns.ptr;
  return PKV_OK;
}

}  // namespace

extern "C" int paged_attention_decode_noalloc(const pkv_layout *layout, float *out, const void *q,
                                              const void *k_pool, const void *v_pool,
                                              const int32_t *d_block_tables, const int32_t *d_context_lens,
                                              int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                              int32_t max_context_len, float scale, const pkv_decode_opts *opts,
                                              void *stream) {
  pkv_decode_args a{};
  const int prep = decode_prepare(layout, out, q, k_pool, v_pool, d_block_tables, d_context_lens, num_seqs,
                                  num_q_heads, max_blocks_per_seq, max_context_len, scale, opts, stream, &a);
  if (prep) return prep == 1 ? PKV_OK : prep;
  const size_t need = paged_attention_workspace_bytes(layout, num_seqs, num_q_heads, max_context_len, opts);
  if (need > kNoallocBytes)
    return pkv_set_error(PKV_ERR_WORKSPACE, "paged_attention_decode_noalloc: %zu bytes of scratch needed, %zu held",
                         need, kNoallocBytes);
  void *ws = nullptr;
  if (int rc = noalloc_scratch(&ws)) return rc;
  carve_workspace(&a, ws);
  return decode_launch(a, opts, stream);
}

extern "C" int pkv_xcd_weights_from_trace(const int32_t *h_trace, int32_t n_waves, int32_t weights_out[8]) {
  if (!h_trace || !weights_out || n_waves < 0 || n_waves > PKV_TRACE_WAVES)
    return pkv_set_error(PKV_ERR_INVALID, "pkv_xcd_weights_from_trace: bad arguments");
  double chunks[PKV_REGIONS] = {}, ticks[PKV_REGIONS] = {};
  for (int32_t w = 0; w < n_waves; ++w) {
    const int32_t *r = h_trace + PKV_TRACE_INTS * w;
    if (r[1] <= 0 || r[0] < 0 || r[0] >= PKV_REGIONS) continue;
    const uint32_t dt = (uint32_t)r[3] - (uint32_t)r[2];  // the clock's low bits may wrap
    if (dt == 0) continue;
    chunks[r[0]] += r[1];
    ticks[r[0]] += dt;
  }
  double rate[PKV_REGIONS], mean = 0;
  for (int x = 0; x < PKV_REGIONS; ++x) {
    if (ticks[x] <= 0) return pkv_set_error(PKV_ERR_INVALID, "no traced wave on XCD %d", x);
    rate[x] = chunks[x] / ticks[x];
    mean += rate[x] / PKV_REGIONS;
  }
  for (int x = 0; x < PKV_REGIONS; ++x) weights_out[x] = (int32_t)std::lround(1000.0 * rate[x] / mean);
  return PKV_OK;
}

extern "C" int paged_attention_prefill(const pkv_layout *layout, float *out, const void *q, const void *k_pool,
                                       const void *v_pool, const int32_t *d_block_tables,
                                       const int32_t *d_context_lens, const int32_t *d_query_start,
                                       int32_t num_seqs, int32_t num_q_heads, int32_t max_blocks_per_seq,
                                       int32_t max_query_len, int32_t max_context_len, float scale, void *stream) {
  if (int rc = pkv_check_layout(layout)) return rc;
  const int32_t H = layout->num_kv_heads;
  if (layout->kv_dtype == PKV_F32)
    return pkv_set_error(PKV_ERR_INVALID, "paged_attention_prefill needs a bf16, int8 or FP8 cache");
  if (num_seqs < 0) return pkv_set_error(PKV_ERR_INVALID, "num_seqs < 0");
  if (num_q_heads <= 0 || num_q_heads % H != 0)
    return pkv_set_error(PKV_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                         num_q_heads, H);
  if (num_q_heads / H > 16)
    return pkv_set_error(PKV_ERR_INVALID, "query heads per kv head must be <= 16 (got %d)", num_q_heads / H);
  if (max_blocks_per_seq <= 0) return pkv_set_error(PKV_ERR_INVALID, "max_blocks_per_seq must be > 0");
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)PKV_BLOCK_SIZE * max_blocks_per_seq ||
      max_context_len > (1 << 22))
    return pkv_set_error(PKV_ERR_INVALID, "max_context_len %d outside [0, min(16 * max_blocks_per_seq, 2^22)]",
                         max_context_len);
  if (max_query_len < 0 || max_query_len > max_context_len)
    return pkv_set_error(PKV_ERR_INVALID, "max_query_len %d outside [0, max_context_len]", max_query_len);
  if (!std::isfinite(scale)) return pkv_set_error(PKV_ERR_INVALID, "scale is not finite");
  if (num_seqs > 65535 || H > 65535) return pkv_set_error(PKV_ERR_INVALID, "grid too large");
  if (num_seqs == 0 || max_query_len == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !d_block_tables || !d_context_lens || !d_query_start)
    return pkv_set_error(PKV_ERR_INVALID, "paged_attention_prefill: NULL pointer");
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16))
    return pkv_set_error(PKV_ERR_INVALID, "paged_attention_prefill: q, out and pools must be 16-byte aligned");
  pkv_prefill_args a{};
  a.L = layout;
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.tables = d_block_tables;
  a.ctx = d_context_lens;
  a.qstart = d_query_start;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.max_blocks = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.max_query_len = max_query_len;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.stream = stream;
  if (int rc = pkv_launch_prefill_mfma(a)) return hip_fail(rc, "prefill kernel launch");
  return PKV_OK;
}

extern "C" int pkv_swap_copy(const pkv_layout *layout, void *dst_k, void *dst_v, int32_t dst_blocks,
                             const void *src_k, const void *src_v, int32_t src_blocks, const int32_t *d_pairs,
                             int32_t num_pairs, void *stream) {
  if (int rc = pkv_check_layout(layout)) return rc;
  if (num_pairs < 0 || dst_blocks < 0 || src_blocks < 0) return pkv_set_error(PKV_ERR_INVALID, "negative count");
  if (num_pairs == 0) return PKV_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !d_pairs) return pkv_set_error(PKV_ERR_INVALID, "pkv_swap_copy: NULL pointer");
  if (!aligned(dst_k, 16) || !aligned(dst_v, 16) || !aligned(src_k, 16) || !aligned(src_v, 16))
    return pkv_set_error(PKV_ERR_INVALID, "pkv_swap_copy: pools must be 16-byte aligned");
  if (num_pairs > 65535 * 32767) return pkv_set_error(PKV_ERR_INVALID, "too many pairs");
  if (int rc = pkv_launch_swap(layout, dst_k, dst_v, dst_blocks, src_k, src_v, src_blocks, d_pairs, num_pairs, stream))
    return hip_fail(rc, "pkv_swap_copy launch");
  return PKV_OK;
}
