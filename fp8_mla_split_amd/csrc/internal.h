// Internal declarations shared by the library's translation units (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

constexpr int kD = 576;    // KV row: 512 latent + 64 rope columns
constexpr int kDv = 512;   // value = first 512 columns of the row
constexpr int kTile = 32;  // KV tokens per tile (one LDS ring slot)
constexpr int kMaxRows = 65536;
constexpr int kMaxSplitsCombine = 4096;

// Unsigned division by a divisor fixed at launch (Granlund & Montgomery, "Division by
// invariant integers using multiplication"): n / d == (t + ((n - t) >> s1)) >> s2 with
// t = mulhi(n, m), for every 32-bit n.
struct FastDiv {
  uint32_t d, m;
  int s1, s2;
};

inline FastDiv make_fastdiv(uint32_t d) {
  int l = 0;
  while (l < 32 && (1ull << l) < d) ++l;  // ceil(log2 d)
  FastDiv f;
  f.d = d;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 1 ? l - 1 : 0;
  return f;
}

__host__ __device__ inline uint32_t fast_div(uint32_t n, const FastDiv& f) {
  const uint32_t t = (uint32_t)(((uint64_t)n * f.m) >> 32);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

struct DecodeParams {
  const uint8_t* q8;
  const uint8_t* kv;
  const int32_t* page_table;
  const int32_t* seq_lens;
  uint16_t* partial_o;                // fp16 bits, in units of kv_scale
  float* partial_lse;
  int batch, q_tokens, heads, rows;   // rows = q_tokens * heads
  int page_size, max_pages, num_splits, groups;
  int64_t page_bytes;                 // page_size * 576
  int tiles_hint;                     // 32-token tiles per split for the host's maximum length
  FastDiv div_splits, div_groups, div_heads, div_tpp;  // by num_splits, groups, heads, page_size/32
  float c2;                           // q_scale * kv_scale * softmax_scale * log2(e)
  float kv_scale;
  // scales read on the device instead (q_scale_dev[0], kv_scale_dev[0]); c2 is then formed in
  // the kernel with the same double-precision products the host uses
  const float* q_scale_dev;
  const float* kv_scale_dev;
  float softmax_scale;
  // per-request query-token counts (NULL: every request has q_tokens); device values are
  // clamped to [0, q_tokens]
  const int32_t* q_lens;
  // per-request count of context positions after the ones this call sees (NULL: none); device
  // values are clamped to [0, q_tokens], which already makes every position visible
  const int32_t* ctx_after;
  // the order in which requests' workgroups are dispatched (a permutation of [0, B); NULL:
  // request order)
  const int32_t* order;
};

// c2 from the three scales: products in double, one rounding to float (host and device alike)
__host__ __device__ inline float score_scale_log2(float q_scale, float kv_scale, float sm_scale) {
  return (float)((double)q_scale * kv_scale * sm_scale * 1.4426950408889634);
}

// Every launch helper below starts here: it drops the thread's last HIP error, so that the
// error it returns after its launches is theirs and not one left by an earlier, unrelated call.
inline void clear_last_error() { (void)hipGetLastError(); }

// The decode call's argument checks other than those of the partial buffers (no HIP call);
// MLA_OK with batch == 0 means there is nothing to do.
mla_status decode_check_args(const uint8_t* q8_dev, const uint8_t* kv_pool_dev,
                             const int32_t* page_table_dev, const int32_t* seq_lens_dev,
                             const int32_t* q_lens_dev, const int32_t* ctx_after_dev,
                             const int32_t* order_dev, int batch, int q_tokens, int heads,
                             int page_size, int max_pages, int max_seq_len, float q_scale,
                             float kv_scale, const float* q_scale_dev,
                             const float* kv_scale_dev, float softmax_scale, int num_splits,
                             int rows_per_group);

hipError_t launch_quantize(const float* src, uint8_t* dst, int64_t n, float scale, hipStream_t s);
int64_t dynamic_quantize_workspace_bytes();
hipError_t launch_quantize_dynamic(const void* src, bool bf16, uint8_t* dst, int64_t n,
                                   float* scale_out, void* workspace, hipStream_t s);
// rope_cos / rope_sin: NULL (no rotation) or fp32 [rope_positions, 32] tables of the rope
// pairs' angles per position.
hipError_t launch_kv_append(const void* src, bool bf16, uint8_t* pool, int64_t num_pages,
                            const int32_t* page_table, const int32_t* seq_lens, int batch,
                            int t_new, int page_size, int max_pages, float scale,
                            const float* rope_cos, const float* rope_sin, int64_t rope_positions,
                            hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int rows_per_group, hipStream_t s);
hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* out, int grid,
                             hipStream_t s);
int64_t read_probe_chunk_bytes();
// v_scale_dev: NULL, or a device float that replaces v_scale.  partial_out: write fp16
// partials (KV-scale units) + lse at rows b * out_b_stride + r instead of bf16 output.
hipError_t launch_combine(const uint16_t* po, const float* pl, int batch, int splits, int rows,
                          float v_scale, const float* v_scale_dev, uint16_t* out, float* out_lse,
                          int64_t out_b_stride, bool partial_out, hipStream_t s);

}  // namespace mla
