// Device-side helpers for the gfx950 kernels: element conversions, DPP
// row reductions, MFMA operand types and the decode kernel parameter block.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Parameters of the decode partition kernels (passed by value).
struct DecodeParams {
  float *out;             // [B][Hq][D]
  const void *q;          // [B][Hq][D]
  const void *k_pool;
  const void *v_pool;
  const int32_t *tables;  // [B][max_blocks]
  const int32_t *ctx;     // [B]
  float *ws_o;            // [B][Hq][num_parts][D]
  float *ws_ml;           // [B][Hq][num_parts][2]
  int32_t num_blocks;
  int32_t H;              // kv heads
  int32_t Hq;             // query heads
  int32_t G;              // Hq / H
  int32_t max_blocks;
  int32_t max_ctx;         // caller's bound on every length (sizes the grid)
  int32_t part_tokens;
  int32_t num_parts;
  float scale_log2;
};

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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
