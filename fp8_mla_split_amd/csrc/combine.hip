// Log-sum-exp merge of split-KV partials -> bf16 output.
//
// The faster split-KV reduction item of the MLA section of the arex-research.com Vera Rubin /
// Kimi K3 write-up replaces a merge that loaded one partial, waited for it, then loaded the
// next (one cache latency per partial) by one that issues every partial's load first and then
// accumulates from registers.  Here each wavefront owns half of one output row (256 of the 512
// value columns, 4 per lane); it reads the row's S log-sum-exps (wave-uniform addresses, so
// the compiler uses scalar loads), then, in batches of 16 splits, issues all 16 partial loads
// before it touches any of them.
//
//   M = max_s lse_s;  w_s = exp(lse_s - M);  O = sum_s w_s O_s / sum_s w_s;  lse = M + log sum w_s
//
// Splits whose lse is -inf contribute nothing and their partial values are never used as
// a weight (their memory may hold anything).  Memory-bound: B*S*R*(512+1)*4 bytes read.
#include "internal.h"

namespace mla {
namespace {

constexpr int kBatch = 16;  // partial loads in flight per lane

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(0x7FC0u | ((u >> 16) & 0x8000u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ __launch_bounds__(64) void combine_kernel(const float* __restrict__ po,
                                                     const float* __restrict__ pl, int S, int R,
                                                     uint16_t* __restrict__ out,
                                                     float* __restrict__ out_lse) {
  const int row = blockIdx.x >> 1;  // b * R + r
  const int half = blockIdx.x & 1;
  const int b = row / R, r = row - b * R;
  const int col = half * 256 + 4 * threadIdx.x;

  const float* lse = pl + (int64_t)b * S * R + r;                  // stride R over splits
  const float* o = po + ((int64_t)b * S * R + r) * kDv + col;     // stride R*512 over splits
  const int64_t ostride = (int64_t)R * kDv;

  float m = -INFINITY;
  for (int s = 0; s < S; ++s) m = fmaxf(m, lse[(int64_t)s * R]);

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int s0 = 0; s0 < S; s0 += kBatch) {
      float4 v[kBatch];
      float w[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {  // issue every load of the batch first
        const int s = s0 + j < S ? s0 + j : S - 1;
        v[j] = *(const float4*)(o + (int64_t)s * ostride);
        w[j] = lse[(int64_t)s * R];
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {  // then accumulate from registers
        const float e = (s0 + j < S && w[j] != -INFINITY) ? __expf(w[j] - m) : 0.f;
        wsum += e;
        acc.x = e != 0.f ? fmaf(e, v[j].x, acc.x) : acc.x;
        acc.y = e != 0.f ? fmaf(e, v[j].y, acc.y) : acc.y;
        acc.z = e != 0.f ? fmaf(e, v[j].z, acc.z) : acc.z;
        acc.w = e != 0.f ? fmaf(e, v[j].w, acc.w) : acc.w;
      }
    }
  }
  const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
  ushort4 h;
  h.x = bf16_rne(acc.x * inv);
  h.y = bf16_rne(acc.y * inv);
  h.z = bf16_rne(acc.z * inv);
  h.w = bf16_rne(acc.w * inv);
  *(ushort4*)(out + (int64_t)row * kDv + col) = h;
  if (out_lse != nullptr && half == 0 && threadIdx.x == 0)
    out_lse[row] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
}

}  // namespace

hipError_t launch_combine(const float* po, const float* pl, int batch, int splits, int rows,
                          uint16_t* out, float* out_lse, hipStream_t s) {
  const int64_t blocks = (int64_t)batch * rows * 2;
  combine_kernel<<<(unsigned)blocks, 64, 0, s>>>(po, pl, splits, rows, out, out_lse);
  return hipGetLastError();
}

}  // namespace mla
