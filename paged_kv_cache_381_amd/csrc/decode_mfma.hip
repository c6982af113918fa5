// PagedAttention decode, matrix-core kernel (bf16 KV, one GQA group per
// workgroup).
//
// What it computes [KV Cache 工程学 §15.5; 新一代 KV Cache 管理 §8.1]: for a
// sequence b and its query heads h of kv group g, the new token's query is
// dotted with the K of every cached token, found by reading block-table entry
// j/16 and slot j%16; a softmax over the whole context weights the cached V.
// The context is cut into partitions of part_tokens tokens; each workgroup
// handles one (partition, kv head, sequence) and keeps a running maximum and
// sum (online softmax), so the softmax stays global even though the data is
// visited block by block (the per-page softmax of the vendor article
// [PagedAttention：大模型KV Cache内存管理革新 §3.2] is not used).
//
// gfx950 mapping.  The G query heads of a group share every K and V tile, so
// the group-by-block products are small dense contractions and run on
// v_mfma_f32_16x16x32_bf16, with the G heads padded to 16 columns:
//   S^T[32 tokens x 16 heads] = K[32 x D] . Q^T[D x 16]   (two 16-row MFMAs)
//   O^T[D x 16 heads]        += V^T[D x 32] . P^T[32 x 16] (D/16 MFMAs)
// One wave consumes a chunk of two 16-token blocks (32 tokens) per step.
// Lane (c = lane%16, j = lane/16) receives S for head c and tokens
// {8(j%2) + 0..3} (first MFMA) and {8(j%2) + 4..7} (second MFMA) of block
// j/2 -- exactly the eight token slots it must hand to the PV MFMA, whose V^T
// operand for lane (d, j) is then 16 contiguous bytes of the [D][16] V tile
// (tokens 8(j%2)..+7 of block j/2).  No cross-lane shuffle sits between the
// two contractions; the softmax needs only two xor-shuffles per chunk (max
// over the four lane groups).  The Q rows of the group are staged once in LDS
// and read into MFMA operands by every wave; the W waves of a workgroup split
// the partition's chunks and are merged through LDS at the end.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace {

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

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

template <int D, int W>
__global__ __launch_bounds__(64 * W) void decode_mfma_kernel(DecodeParams P) {
  constexpr int NKK = D / 32;  // score MFMAs per 16-row token set
  constexpr int NNN = D / 16;  // PV MFMAs
  constexpr int CPR = D / 8;   // 16-byte K chunks per token (8 bf16 each)
  extern __shared__ __align__(16) char smem[];
  uint4 *q_lds = reinterpret_cast<uint4 *>(smem);                  // [16][CPR]
  float *red_m = reinterpret_cast<float *>(smem + 16 * CPR * 16);  // [W][16]
  float *red_l = red_m + W * 16;                                    // [W][16]
  float *red_o = red_l + W * 16;                                    // [W][G][D]

  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = P.G;
  const int n = clamp_len(P.ctx[b], P.max_blocks, P.max_ctx);
  const int t0 = part * P.part_tokens;
  float *out_bg = P.out + ((size_t)b * P.Hq + (size_t)g * G) * D;
  if (n == 0) {
    if (part == 0)
      for (int i = tid; i < G * D; i += 64 * W) out_bg[i] = 0.f;
    return;
  }
  if (t0 >= n) return;
  const int t1 = min(t0 + P.part_tokens, n);
  const int nchunks = (t1 - t0 + 31) >> 5;
  const int nparts_b = (n + P.part_tokens - 1) / P.part_tokens;

  const uint16_t *qg = reinterpret_cast<const uint16_t *>(P.q) + ((size_t)b * P.Hq + (size_t)g * G) * D;
  for (int i = tid; i < 16 * CPR; i += 64 * W) {
    const int h = i / CPR, c = i - h * CPR;
    q_lds[i] = h < G ? *reinterpret_cast<const uint4 *>(qg + (size_t)h * D + c * 8) : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  const int r16 = lane & 15, grp = lane >> 4;
  bf16x8_t qb[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qb[kk] = as_bf16x8(q_lds[r16 * CPR + 4 * kk + grp]);

  // Row r16 of the score MFMAs holds a token of block (r16 >> 3); see header.
  const int ksel = r16 >> 3;
  const int ktx = ((r16 >> 2) & 1) * 8 + (r16 & 3);
  const int vsel = grp >> 1, vhalf = grp & 1;

  f32x4_t o[NNN];
#pragma unroll
  for (int nn = 0; nn < NNN; ++nn) o[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  const int32_t *tbl = P.tables + (size_t)b * P.max_blocks;
  const uint16_t *kpool = reinterpret_cast<const uint16_t *>(P.k_pool);
  const uint16_t *vpool = reinterpret_cast<const uint16_t *>(P.v_pool);
  constexpr size_t TILE = (size_t)16 * D;

  for (int ch = w; ch < nchunks; ch += W) {
    const int tok0 = t0 + ch * 32;
    const int jA = tok0 >> 4;
    const int physA = clamp_block(tbl[jA], P.num_blocks);
    const int physB = (tok0 + 16 < n) ? clamp_block(tbl[jA + 1], P.num_blocks) : physA;
    const size_t tA = ((size_t)physA * P.H + g) * TILE, tB = ((size_t)physB * P.H + g) * TILE;
    const uint4 *kt = reinterpret_cast<const uint4 *>(kpool + (ksel ? tB : tA));
    const uint4 *vt = reinterpret_cast<const uint4 *>(vpool + (vsel ? tB : tA));

    uint4 ax[NKK], ay[NKK], va[NNN];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int c = 4 * kk + grp;
      ax[kk] = kt[c * 16 + ktx];
      ay[kk] = kt[c * 16 + ktx + 4];
    }
#pragma unroll
    for (int nn = 0; nn < NNN; ++nn) va[nn] = vt[2 * (16 * nn + r16) + vhalf];

    f32x4_t sx = {0.f, 0.f, 0.f, 0.f}, sy = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      sx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ax[kk]), qb[kk], sx, 0, 0, 0);
      sy = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ay[kk]), qb[kk], sy, 0, 0, 0);
    }
    const int tb = tok0 + 16 * (grp >> 1) + 8 * (grp & 1);
    float s[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s[r] = (tb + r < n) ? sx[r] * P.scale_log2 : -INFINITY;
      s[4 + r] = (tb + 4 + r < n) ? sy[r] * P.scale_log2 : -INFINITY;
    }
    float cmax = s[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) cmax = fmaxf(cmax, s[r]);
    cmax = rows_max4(cmax);
    const float mnew = fmaxf(m, cmax);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    bf16x8_t pv;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const __bf16 pr = (__bf16)fast_exp2(s[r] - mnew);
      pv[r] = pr;
      psum += (float)pr;  // the PV numerator uses the rounded weights too
    }
    l = l * alpha + psum;
#pragma unroll
    for (int nn = 0; nn < NNN; ++nn) o[nn] *= alpha;
    if (tok0 + 32 > n) {  // slots past the context may hold anything, NaN included
      const int nvalid = min(max(n - (tok0 + 16 * vsel + 8 * vhalf), 0), 8);
#pragma unroll
      for (int nn = 0; nn < NNN; ++nn) va[nn] = keep_first(va[nn], nvalid);
    }
#pragma unroll
    for (int nn = 0; nn < NNN; ++nn) o[nn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va[nn]), pv, o[nn], 0, 0, 0);
  }

  l = rows_sum4(l);
  if (grp == 0) {
    red_m[w * 16 + r16] = m;
    red_l[w * 16 + r16] = l;
  }
  if (r16 < G) {
#pragma unroll
    for (int nn = 0; nn < NNN; ++nn)
#pragma unroll
      for (int r = 0; r < 4; ++r) red_o[((size_t)w * G + r16) * D + 16 * nn + 4 * grp + r] = o[nn][r];
  }
  __syncthreads();

  for (int i = tid; i < G * D; i += 64 * W) {
    const int h = i / D, d = i - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < W; ++v) M = fmaxf(M, red_m[v * 16 + h]);
    float acc = 0.f, L = 0.f;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const float f = fast_exp2(red_m[v * 16 + h] - M);
      acc += f * red_o[((size_t)v * G + h) * D + d];
      L += f * red_l[v * 16 + h];
    }
    if (nparts_b == 1) {
      out_bg[(size_t)h * D + d] = acc / L;
    } else {
      const size_t row = ((size_t)b * P.Hq + (size_t)g * G + h) * P.num_parts + part;
      P.ws_o[row * D + d] = acc;
      if (d == 0) {
        P.ws_ml[2 * row] = M;
        P.ws_ml[2 * row + 1] = L;
      }
    }
  }
}

constexpr int kWaves = 4;

template <int D>
int launch(const pkv_decode_args &a, const DecodeParams &p) {
  const size_t lds = 16 * (D / 8) * 16 + (size_t)(2 * kWaves * 16 + kWaves * p.G * D) * sizeof(float);
  dim3 grid(a.num_parts, a.L->num_kv_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_mfma_kernel<D, kWaves>), grid, dim3(64 * kWaves), lds,
                     reinterpret_cast<hipStream_t>(a.stream), p);
  return (int)hipGetLastError();
}

}  // namespace

int pkv_launch_decode_mfma(const pkv_decode_args &a) {
  DecodeParams p{a.out, a.q, a.k_pool, a.v_pool, a.tables, a.ctx, a.ws_o, a.ws_ml,
                 a.L->num_blocks, a.L->num_kv_heads, a.num_q_heads, a.num_q_heads / a.L->num_kv_heads,
                 a.max_blocks, a.max_ctx, a.part_tokens, a.num_parts, a.scale_log2};
  return a.L->head_dim == 128 ? launch<128>(a, p) : launch<64>(a, p);
}
