// Log-sum-exp merge of split-KV partials -> bf16 output.
//
// The faster split-KV reduction item of the MLA section of the arex-research.com Vera Rubin /
// Kimi K3 write-up replaces a merge that loaded one partial, waited for it, then loaded the
// next (one cache latency per partial) by one that issues every partial's load first and then
// accumulates from registers.  Here a row's 512 value columns are split over kCw workgroups
// (kCw * rows workgroups in all, so a batch-1 merge still spreads over the whole chip); a
// workgroup has NW = ceil(S / (B kCw)) waves (at most 16) and each wave owns B kCw splits per
// batch, with B = 4, 8 or 16 load instructions per batch as S requires.  A lane covers 8
// columns (16 bytes) of one split row, so one wave-wide load instruction fetches kCw split
// rows; a wave issues its whole batch of loads (and the log-sum-exps) before it touches any of
// them, keeps a running max of its splits' lse and rescales as it goes, and the workgroup's
// lanes meet in LDS at the end.
//
//   M = max_s lse_s;  w_s = exp(lse_s - M);  O = v_scale * sum_s w_s O_s / sum_s w_s;
//   lse = M + log sum_s w_s
//
// Partial rows are fp16 values in units of v_scale.  Splits whose lse is -inf contribute
// nothing (their partial rows may hold anything; they are loaded but never used).
// Memory-bound: B*S*R*(1024 + 4) bytes read, B*R*1024 (+ 4) written.
#include "internal.h"

namespace mla {
namespace {

constexpr int kCw = 2;       // workgroups (column chunks) per output row
constexpr int kLanesPerRow = 64 / kCw;  // lanes covering one split row's chunk
constexpr int kMaxWaves = 16;

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)(0x7FC0u | ((u >> 16) & 0x8000u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

struct Partial {
  float m, ws;
  float acc[8];
};

// kBatch: load instructions a wave issues before it accumulates (kBatch * kCw splits).
template <int kBatch>
__global__ __launch_bounds__(64 * kMaxWaves) void combine_kernel(
    const uint16_t* __restrict__ po, const float* __restrict__ pl, int S, int R, float v_scale,
    uint16_t* __restrict__ out, float* __restrict__ out_lse) {
  extern __shared__ Partial red[];  // one entry per thread
  const int row = blockIdx.x / kCw;  // b * R + r
  const int chunk = blockIdx.x - row * kCw;
  const int b = row / R, r = row - b * R;
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sub = lane / kLanesPerRow;             // which of the kCw split rows of a load
  const int pos = lane - sub * kLanesPerRow;       // 16-byte column group within the chunk
  const int col0 = chunk * (kDv / kCw) + 8 * pos;  // first of this lane's 8 columns

  const float* lse = pl + (int64_t)b * S * R + r;                      // stride R over splits
  const uint16_t* o = po + ((int64_t)b * S * R + r) * kDv + col0;      // stride R*512
  const int64_t ostride = (int64_t)R * kDv;

  Partial p;
  p.m = -INFINITY;
  p.ws = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) p.acc[c] = 0.f;

  // split of load j of batch t: ((t * nw + wave) * kBatch + j) * kCw + sub
  for (int s0 = wave * kBatch * kCw; s0 < S; s0 += nw * kBatch * kCw) {
    uint4 v[kBatch];
    float l[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {  // every load of the batch first
      const int s = s0 + j * kCw + sub;
      const int sc = min(s, S - 1);
      l[j] = s < S ? lse[(int64_t)sc * R] : -INFINITY;
      v[j] = *(const uint4*)(o + (int64_t)sc * ostride);
    }
    float bm = p.m;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) bm = fmaxf(bm, l[j]);
    if (bm != -INFINITY) {
      const float rescale = __expf(p.m - bm);  // 0 when p.m is -inf
      p.ws *= rescale;
#pragma unroll
      for (int c = 0; c < 8; ++c) p.acc[c] *= rescale;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {  // then accumulate from registers
        const bool live = l[j] != -INFINITY;
        const float e = live ? __expf(l[j] - bm) : 0.f;
        p.ws += e;
        const _Float16* h = (const _Float16*)&v[j];
#pragma unroll
        for (int c = 0; c < 8; ++c) p.acc[c] = fmaf(e, live ? (float)h[c] : 0.f, p.acc[c]);
      }
      p.m = bm;
    }
  }
  red[threadIdx.x] = p;
  __syncthreads();
  if (wave != 0 || sub != 0) return;

  // lane pos of wave 0 merges the nw * kCw partials of its column group
  float M = -INFINITY;
  for (int k = 0; k < nw * kCw; ++k)
    M = fmaxf(M, red[(k / kCw) * 64 + (k % kCw) * kLanesPerRow + pos].m);
  float ws = 0.f, tot[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    for (int k = 0; k < nw * kCw; ++k) {
      const Partial& q = red[(k / kCw) * 64 + (k % kCw) * kLanesPerRow + pos];
      const float sc = __expf(q.m - M);  // 0 for a partial that saw no live split
      ws += sc * q.ws;
#pragma unroll
      for (int c = 0; c < 8; ++c) tot[c] = fmaf(sc, q.acc[c], tot[c]);
    }
  }
  const float f = ws > 0.f ? v_scale / ws : 0.f;
  uint4 packed;
  packed.x = (uint32_t)bf16_rne(tot[0] * f) | ((uint32_t)bf16_rne(tot[1] * f) << 16);
  packed.y = (uint32_t)bf16_rne(tot[2] * f) | ((uint32_t)bf16_rne(tot[3] * f) << 16);
  packed.z = (uint32_t)bf16_rne(tot[4] * f) | ((uint32_t)bf16_rne(tot[5] * f) << 16);
  packed.w = (uint32_t)bf16_rne(tot[6] * f) | ((uint32_t)bf16_rne(tot[7] * f) << 16);
  *(uint4*)(out + (int64_t)row * kDv + col0) = packed;
  if (out_lse != nullptr && chunk == 0 && pos == 0)
    out_lse[row] = ws > 0.f ? M + logf(ws) : -INFINITY;
}

}  // namespace

template <int kBatch>
static void launch_batch(const uint16_t* po, const float* pl, int batch, int splits, int rows,
                         float v_scale, uint16_t* out, float* out_lse, hipStream_t s) {
  const int64_t blocks = (int64_t)batch * rows * kCw;
  int nw = (splits + kBatch * kCw - 1) / (kBatch * kCw);
  nw = nw < 1 ? 1 : (nw > kMaxWaves ? kMaxWaves : nw);
  const size_t lds = sizeof(Partial) * 64 * nw;
  combine_kernel<kBatch><<<(unsigned)blocks, 64 * nw, lds, s>>>(po, pl, splits, rows, v_scale,
                                                                 out, out_lse);
}

hipError_t launch_combine(const uint16_t* po, const float* pl, int batch, int splits, int rows,
                          float v_scale, uint16_t* out, float* out_lse, hipStream_t s) {
  // as many loads in flight per wave as there are splits to cover, up to 16
  if (splits <= 4 * kCw)
    launch_batch<4>(po, pl, batch, splits, rows, v_scale, out, out_lse, s);
  else if (splits <= 8 * kCw)
    launch_batch<8>(po, pl, batch, splits, rows, v_scale, out, out_lse, s);
  else
    launch_batch<16>(po, pl, batch, splits, rows, v_scale, out, out_lse, s);
  return hipGetLastError();
}

}  // namespace mla
