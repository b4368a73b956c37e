// mla_decode_noalloc: split-KV decode and its log-sum-exp combine in one call that allocates
// nothing, for callers that cannot call hipMalloc (work under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  The split partials, which mla_decode_splitkv
// writes into caller buffers, live here in a device array the library owns: one copy per GPU
// (each device that loads the library's code holds its own), kept until the process ends.
//
// Host code never passes the array's name to a kernel or a copy: in host code that name is a
// stand-in, not a device address.  Its address on the current device is looked up once per
// device with hipGetSymbolAddress and kept; the kernels (the same decode and combine kernels
// the other entry points launch) take that address as their partial buffers.
//
// Nothing in the array has to start at zero: the decode writes every partial lse entry of
// the (request, split, row) range it covers (-inf for an empty chunk or a row that sees no
// position) before the combine reads it, and the combine never uses a partial output whose
// lse is -inf.  Every call on one GPU uses the same array, so calls that overlap in time on
// one GPU (different streams, host threads) race; calls on one stream are ordered.
#include <mutex>

#include "internal.h"
#include "mla.h"

namespace {

constexpr int64_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
constexpr int64_t kRowBytes = mla::kDv * 2 + 4;  // fp16 partial row + its lse
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

uint8_t* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// The array's device address on the current device, looked up on the first call there.  The
// kernels run on the stream's device, so a stream of another device is refused (its kernels
// would be handed this device's address).
mla_status scratch_on_current_device(hipStream_t stream, uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return MLA_ERR_HIP;
    if (sdev != dev) return MLA_ERR_INVALID_ARG;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch[dev] = (uint8_t*)ptr;
  });
  if (g_scratch_err[dev] != hipSuccess || g_scratch[dev] == nullptr) return MLA_ERR_HIP;
  *out = g_scratch[dev];
  return MLA_OK;
}

// wanted if the partials of that many splits fit the array, else 0.
int64_t splits_that_fit(int64_t rows_per_split, int64_t wanted) {
  const int64_t most = (kScratchBytes - 256) / (rows_per_split * kRowBytes);
  return wanted <= most ? wanted : 0;
}

}  // namespace

extern "C" mla_status mla_decode_noalloc(const uint8_t* q8_dev, const uint8_t* kv_pool_dev,
                                         const int32_t* page_table_dev,
                                         const int32_t* seq_lens_dev, int batch, int q_tokens,
                                         int heads, int page_size, int max_pages,
                                         int max_seq_len, float q_scale, float kv_scale,
                                         float softmax_scale, int num_splits,
                                         uint16_t* out_bf16_dev, float* out_lse_dev,
                                         void* stream) {
  // every argument check first (no HIP call before them)
  const mla_status chk = mla::decode_check_args(
      q8_dev, kv_pool_dev, page_table_dev, seq_lens_dev, nullptr, nullptr, nullptr, batch,
      q_tokens, heads, page_size, max_pages, max_seq_len, q_scale, kv_scale, nullptr, nullptr,
      softmax_scale, num_splits, 0);
  if (chk != MLA_OK || batch == 0) return chk;
  if (out_bf16_dev == nullptr) return MLA_ERR_INVALID_ARG;
  const int64_t rows_per_split = (int64_t)batch * q_tokens * heads;  // B * Sq * H
  int64_t S = num_splits;
  if (S > 0) {
    if (splits_that_fit(rows_per_split, S) == 0) return MLA_ERR_WORKSPACE;
  } else {
    if (splits_that_fit(rows_per_split, 1) == 0) return MLA_ERR_WORKSPACE;
    int planned = 1;
    const mla_status st = mla_splitkv_plan(batch, q_tokens, heads, max_seq_len, 0, 0, &planned,
                                           nullptr, nullptr);
    if (st != MLA_OK) return st;
    S = planned;
    while (S > 1 && splits_that_fit(rows_per_split, S) == 0) --S;
  }
  uint8_t* base = nullptr;
  const mla_status sst = scratch_on_current_device((hipStream_t)stream, &base);
  if (sst != MLA_OK) return sst;
  // partial outputs first, their lse after them (256-byte aligned)
  const int64_t entries = rows_per_split * S;
  uint16_t* po = (uint16_t*)base;
  float* pl = (float*)(base + ((entries * mla::kDv * 2 + 255) / 256) * 256);
  const mla_status d = mla_decode_splitkv(q8_dev, kv_pool_dev, page_table_dev, seq_lens_dev,
                                          batch, q_tokens, heads, page_size, max_pages,
                                          max_seq_len, q_scale, kv_scale, softmax_scale, (int)S,
                                          128, po, pl, entries, stream);
  if (d != MLA_OK) return d;
  return mla_splitkv_combine(po, pl, batch, (int)S, q_tokens, heads, kv_scale, out_bf16_dev,
                             out_lse_dev, stream);
}
