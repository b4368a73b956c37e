// Internal declarations shared by the library's translation units (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kD = 576;    // KV row: 512 latent + 64 rope columns
constexpr int kDv = 512;   // value = first 512 columns of the row
constexpr int kTile = 32;  // KV tokens per tile (one LDS ring slot)
constexpr int kMaxRows = 65536;
constexpr int kMaxSplitsCombine = 4096;

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
  float c2;                           // q_scale * kv_scale * softmax_scale * log2(e)
  float kv_scale;
};

hipError_t launch_quantize(const float* src, uint8_t* dst, int64_t n, float scale, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int rows_per_group, hipStream_t s);
hipError_t launch_combine(const uint16_t* po, const float* pl, int batch, int splits, int rows,
                          float v_scale, uint16_t* out, float* out_lse, hipStream_t s);

}  // namespace mla
