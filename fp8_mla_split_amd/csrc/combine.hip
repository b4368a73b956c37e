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
// them, and keeps a running max of its splits' lse, rescaling as it goes.  At the end the two
// halves of each wave merge across lanes in registers, and the waves (if more than one) meet
// in LDS, where wave 0 merges their entries, again half in each lane half.
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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Partial {
  float m, ws;
  float acc[8];
};

// (m, ws, acc) of a and b merged into a: both rescaled to the larger m.  A side that saw no
// live split (m = -inf) contributes nothing; two such sides stay empty.
__device__ __forceinline__ void merge_into(Partial& a, const Partial& b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return;
  const float sa = __expf(a.m - M), sb = __expf(b.m - M);  // exp(-inf) = 0
  a.ws = sa * a.ws + sb * b.ws;
#pragma unroll
  for (int c = 0; c < 8; ++c) a.acc[c] = sa * a.acc[c] + sb * b.acc[c];
  a.m = M;
}

// The partials of lanes l mod 32 (lo) and l mod 32 + 32 (hi), in every lane: one
// v_permlane32_swap per value, whose two results are those two lanes' values in either half.
__device__ __forceinline__ void lane_halves(const Partial& p, Partial& lo, Partial& hi) {
  const float* src = &p.m;
  float* dlo = &lo.m;
  float* dhi = &hi.m;
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(src[i]),
                                                    __float_as_uint(src[i]), false, false);
    dlo[i] = __uint_as_float(r[0]);
    dhi[i] = __uint_as_float(r[1]);
  }
}

// Both halves of the wave end up holding the merge of lanes l mod 32 and l mod 32 + 32.
__device__ __forceinline__ void merge_halves(Partial& p) {
  Partial hi;
  lane_halves(p, p, hi);
  merge_into(p, hi);
}

// Column group pos of the nw per-wave entries in LDS, merged: lane half h takes entries
// h, h + 2, h + 4, ... (merge_halves then joins the two halves).  Every read is unconditional
// (an index past nw reads entry nw - 1, which is then ignored), so all of them are in flight
// together.
__device__ __forceinline__ Partial merge_entries(const Partial* red, int nw, int pos, int h) {
  Partial e[kMaxWaves / 2];
#pragma unroll
  for (int k = 0; k < kMaxWaves / 2; ++k) e[k] = red[min(2 * k + h, nw - 1) * kLanesPerRow + pos];
  Partial q;
  q.m = -INFINITY;
  q.ws = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) q.acc[c] = 0.f;
#pragma unroll
  for (int k = 0; k < kMaxWaves / 2; ++k)
    if (2 * k + h < nw) q.m = fmaxf(q.m, e[k].m);
  if (q.m == -INFINITY) return q;
#pragma unroll
  for (int k = 0; k < kMaxWaves / 2; ++k) {
    // 0 for an entry past nw or one that saw no live split
    const float sc = 2 * k + h < nw ? __expf(e[k].m - q.m) : 0.f;
    q.ws = fmaf(sc, e[k].ws, q.ws);
#pragma unroll
    for (int c = 0; c < 8; ++c) q.acc[c] = fmaf(sc, e[k].acc[c], q.acc[c]);
  }
  return q;
}

// kBatch: load instructions a wave issues before it accumulates (kBatch * kCw splits).
// kPartialOut: instead of the bf16 output, write the merged result as one partial in the
// decode's own format (fp16 in units of the KV scale, natural-log lse) at row
// b * out_b_stride + r, so that a further combine can merge it with others (the partials of
// other context shards, say); out_lse is then required and v_scale unused.
template <int kBatch, bool kPartialOut>
__global__ __launch_bounds__(64 * kMaxWaves) void combine_kernel(
    const uint16_t* __restrict__ po, const float* __restrict__ pl, int S, int R, int nw,
    float v_scale, const float* __restrict__ v_scale_dev, uint16_t* __restrict__ out,
    float* __restrict__ out_lse, int64_t out_b_stride) {
  static_assert(kCw == 2, "the two split rows of a load sit in lanes l and l + 32");
  // all arguments in one batch of scalar loads (one trip to the argument memory)
  asm volatile("" ::"s"(po), "s"(pl), "s"(S), "s"(R), "s"(nw), "s"(v_scale), "s"(out),
               "s"(out_lse), "s"(v_scale_dev));
  // a scale kept on the device (written by an earlier kernel on the stream) replaces v_scale
  if (v_scale_dev != nullptr)
    v_scale = *(const __attribute__((address_space(4))) float*)v_scale_dev;
  extern __shared__ Partial red[];  // one entry per (wave, column group)
  const int row = blockIdx.x / kCw;  // b * R + r
  const int chunk = blockIdx.x - row * kCw;
  const int b = row / R, r = row - b * R;
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
    u32x4 v[kBatch];
    float l[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {  // every load of the batch first
      const int s = s0 + j * kCw + sub;
      const int sc = min(s, S - 1);
      l[j] = lse[(int64_t)sc * R];  // loaded unconditionally (no branch per load)
      v[j] = *(const u32x4*)(o + (int64_t)sc * ostride);
    }
    // every load of the batch is in flight before the first is used (the compiler would
    // otherwise sink them into the accumulation below, one round trip each)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) asm volatile("" ::"v"(l[j]), "v"(v[j]));
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (s0 + j * kCw + sub >= S) l[j] = -INFINITY;
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
  // lanes l and l + 32 hold the same columns of different splits: merge them in registers;
  // with several waves, these meet in LDS and wave 0 merges their entries
  merge_halves(p);
  if (nw > 1) {
    if (lane < kLanesPerRow) red[wave * kLanesPerRow + pos] = p;
    __syncthreads();
    if (wave != 0) return;
    p = merge_entries(red, nw, pos, lane >> 5);
    merge_halves(p);
  }
  if (lane >= kLanesPerRow) return;
  const float ws = p.ws, M = p.m;
  const float* tot = p.acc;
  if constexpr (kPartialOut) {
    const float f = ws > 0.f ? 1.0f / ws : 0.f;  // |O| <= 448 in units of the KV scale
    const int64_t orow = (int64_t)b * out_b_stride + r;
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 h = {(_Float16)(tot[0] * f), (_Float16)(tot[1] * f), (_Float16)(tot[2] * f),
                  (_Float16)(tot[3] * f), (_Float16)(tot[4] * f), (_Float16)(tot[5] * f),
                  (_Float16)(tot[6] * f), (_Float16)(tot[7] * f)};
    *(uint4*)(out + orow * kDv + col0) = __builtin_bit_cast(uint4, h);
    if (chunk == 0 && pos == 0) out_lse[orow] = ws > 0.f ? M + logf(ws) : -INFINITY;
    return;
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
                         float v_scale, const float* v_scale_dev, uint16_t* out, float* out_lse,
                         int64_t out_b_stride, bool partial_out, hipStream_t s) {
  const int64_t blocks = (int64_t)batch * rows * kCw;
  int nw = (splits + kBatch * kCw - 1) / (kBatch * kCw);
  nw = nw < 1 ? 1 : (nw > kMaxWaves ? kMaxWaves : nw);
  const size_t lds = sizeof(Partial) * kLanesPerRow * nw;
  if (partial_out)
    combine_kernel<kBatch, true><<<(unsigned)blocks, 64 * nw, lds, s>>>(
        po, pl, splits, rows, nw, v_scale, v_scale_dev, out, out_lse, out_b_stride);
  else
    combine_kernel<kBatch, false><<<(unsigned)blocks, 64 * nw, lds, s>>>(
        po, pl, splits, rows, nw, v_scale, v_scale_dev, out, out_lse, out_b_stride);
}

hipError_t launch_combine(const uint16_t* po, const float* pl, int batch, int splits, int rows,
                          float v_scale, const float* v_scale_dev, uint16_t* out, float* out_lse,
                          int64_t out_b_stride, bool partial_out, hipStream_t s) {
  clear_last_error();
  // As many loads in flight per wave as there are splits to cover, up to 16; from 64 splits
  // on, 8 per wave and twice the waves (up to 16) spread the loads wider (measured on MI355X:
  // 6.2 instead of 6.5 us at 256 splits, 3.9 instead of 4.4 at 64).
  if (splits <= 4 * kCw)
    launch_batch<4>(po, pl, batch, splits, rows, v_scale, v_scale_dev, out, out_lse, out_b_stride,
                    partial_out, s);
  else if (splits <= 8 * kCw || splits >= 64)
    launch_batch<8>(po, pl, batch, splits, rows, v_scale, v_scale_dev, out, out_lse, out_b_stride,
                    partial_out, s);
  else
    launch_batch<16>(po, pl, batch, splits, rows, v_scale, v_scale_dev, out, out_lse, out_b_stride,
                    partial_out, s);
  return hipGetLastError();
}

}  // namespace mla
