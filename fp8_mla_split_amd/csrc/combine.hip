// Log-sum-exp merge of split-KV partials -> bf16 output.
//
// The faster split-KV reduction item of the MLA section of the arex-research.com Vera Rubin /
// Kimi K3 write-up replaces a merge that loaded one partial, waited for it, then loaded the
// next (one cache latency per partial) by one that issues every partial's load first and then
// accumulates from registers.  Here one workgroup (four waves) owns one output row; each lane
// owns 8 of its 512 value columns, and wave w takes the splits s = w, w + 4, ...  A wave reads
// the row's S log-sum-exps, then, in batches of 16 splits, issues all 16 partial-row loads
// (16 bytes per lane, one 1 KiB row per instruction) before it touches any of them.  The
// four waves' sums meet in LDS.
//
//   M = max_s lse_s;  w_s = exp(lse_s - M);  O = v_scale * sum_s w_s O_s / sum_s w_s;
//   lse = M + log sum_s w_s
//
// Partial rows are fp16 values in units of v_scale.  Splits whose lse is -inf contribute
// nothing and their partial rows are never read (their memory may hold anything).
// Memory-bound: B*S*R*(1024 + 4) bytes read.
#include "internal.h"

namespace mla {
namespace {

constexpr int kBatch = 16;  // partial rows in flight per wave

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(0x7FC0u | ((u >> 16) & 0x8000u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ po,
                                                      const float* __restrict__ pl, int S, int R,
                                                      float v_scale, uint16_t* __restrict__ out,
                                                      float* __restrict__ out_lse) {
  __shared__ float red_m[4];
  __shared__ float red_w[4];
  __shared__ float4 red_o[4][64][2];
  const int row = blockIdx.x;  // b * R + r
  const int b = row / R, r = row - b * R;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  const float* lse = pl + (int64_t)b * S * R + r;                       // stride R over splits
  const uint16_t* o = po + ((int64_t)b * S * R + r) * kDv + 8 * lane;   // stride R*512
  const int64_t ostride = (int64_t)R * kDv;

  // row max of the lse over all splits
  float m = -INFINITY;
  for (int s = threadIdx.x; s < S; s += 256) m = fmaxf(m, lse[(int64_t)s * R]);
  m = wave_max(m);
  if (lane == 0) red_m[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int s0 = wave; s0 < S; s0 += 4 * kBatch) {
      uint4 v[kBatch];
      float w[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {  // issue every load of the batch first
        const int s = min(s0 + 4 * j, S - 1);
        w[j] = s0 + 4 * j < S ? lse[(int64_t)s * R] : -INFINITY;
        v[j] = *(const uint4*)(o + (int64_t)s * ostride);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {  // then accumulate from registers
        if (w[j] == -INFINITY) continue;  // wave-uniform: an empty split is never read
        const float e = __expf(w[j] - m);
        wsum += e;
        const _Float16* h = (const _Float16*)&v[j];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = fmaf(e, (float)h[c], acc[c]);
      }
    }
  }
  red_o[wave][lane][0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  red_o[wave][lane][1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  if (lane == 0) red_w[wave] = wsum;
  __syncthreads();
  if (wave != 0) return;
  float tot[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float ws = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 a = red_o[k][lane][0], c = red_o[k][lane][1];
    tot[0] += a.x; tot[1] += a.y; tot[2] += a.z; tot[3] += a.w;
    tot[4] += c.x; tot[5] += c.y; tot[6] += c.z; tot[7] += c.w;
    ws += red_w[k];
  }
  const float f = ws > 0.f ? v_scale / ws : 0.f;
  uint4 packed;
  packed.x = (uint32_t)bf16_rne(tot[0] * f) | ((uint32_t)bf16_rne(tot[1] * f) << 16);
  packed.y = (uint32_t)bf16_rne(tot[2] * f) | ((uint32_t)bf16_rne(tot[3] * f) << 16);
  packed.z = (uint32_t)bf16_rne(tot[4] * f) | ((uint32_t)bf16_rne(tot[5] * f) << 16);
  packed.w = (uint32_t)bf16_rne(tot[6] * f) | ((uint32_t)bf16_rne(tot[7] * f) << 16);
  *(uint4*)(out + (int64_t)row * kDv + 8 * lane) = packed;
  if (out_lse != nullptr && lane == 0) out_lse[row] = ws > 0.f ? m + logf(ws) : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const uint16_t* po, const float* pl, int batch, int splits, int rows,
                          float v_scale, uint16_t* out, float* out_lse, hipStream_t s) {
  const int64_t blocks = (int64_t)batch * rows;
  combine_kernel<<<(unsigned)blocks, 256, 0, s>>>(po, pl, splits, rows, v_scale, out, out_lse);
  return hipGetLastError();
}

}  // namespace mla
