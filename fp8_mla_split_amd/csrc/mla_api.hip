// Host side of libmla.so: argument checks (all before any HIP call), the split planner, the
// per-device compute-unit cache and the kernel launches.  See include/mla.h for the contract.
#include <math.h>
#include <mutex>

#include "internal.h"
#include "mla.h"

namespace {

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];
std::once_flag g_cu_once[kMaxDevices];

mla_status device_cu_count(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
  std::call_once(g_cu_once[dev], [dev] {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) v = 0;
    g_cu_count[dev] = v;
  });
  if (g_cu_count[dev] <= 0) return MLA_ERR_HIP;
  *out = g_cu_count[dev];
  return MLA_OK;
}

bool good_scale(float s) { return isfinite(s) && s > 0.0f; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Planner cost model, in microseconds, with rates measured on MI355X for the decode kernel
// (one workgroup per CU; a 64-token step of 128 query rows takes ~2.8 us) plus the traffic
// of the split partials (written by the decode kernel, read back by the combine).  A request
// of L tokens is cut into S chunks of ceil(ceil(L/64) / S) steps.  The hardware hands
// workgroups to CUs as CUs free up, so the decode takes about the longer of the longest
// chunk and the total work spread over the CUs; total_tokens (the sum of the requests'
// lengths) is B * L_max when every request is as long as the longest.
constexpr double kStepUs = 2.8;             // one 64-token step of one workgroup
constexpr double kWgOverheadUs = 3.0;       // staging before the first step, epilogue
constexpr double kPartialBytesPerUs = 5e6;  // partial rows written + read back
constexpr double kCombineUs = 3.0;          // the combine launch itself

double plan_cost(int64_t B, int64_t M, int64_t L, int64_t total_tokens, int cu, int64_t S) {
  const int64_t G = cdiv(M, 128);
  const int64_t steps_max = cdiv(cdiv(L, 64), S);  // the longest chunk
  const int64_t total_steps = G * cdiv(total_tokens, 64);
  const int64_t per_cu = cdiv(total_steps, cu);
  const int64_t rounds = cdiv(B * S * G, cu);
  const double t_dec = (double)rounds * kWgOverheadUs +
                       (double)(steps_max > per_cu ? steps_max : per_cu) * kStepUs;
  const double t_part = (double)(B * S * M) * (1024.0 + 4.0) * 2.0 / kPartialBytesPerUs;
  return t_dec + t_part + (S > 1 ? kCombineUs : 0.0);
}

mla_status plan(int batch, int q_tokens, int heads, int max_seq_len, int64_t total_tokens,
                int cu, int* splits, int* rows_per_group) {
  const int64_t M = (int64_t)q_tokens * heads;
  const int64_t tiles = cdiv(max_seq_len, 32);
  const int64_t s_max = tiles / 2 > 0 ? tiles / 2 : 1;  // at least one full step per chunk
  const int64_t total = total_tokens > 0 ? total_tokens : (int64_t)batch * max_seq_len;
  double best = -1.0;
  int best_s = 1;
  for (int64_t S = 1; S <= s_max && S <= 4096; ++S) {
    const double c = plan_cost(batch, M, max_seq_len, total, cu, S);
    if (best < 0.0 || c < best) {
      best = c;
      best_s = (int)S;
    }
  }
  *splits = best_s;
  *rows_per_group = 128;
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: break;
  }
  return "MLA_ERR_UNKNOWN";
}

mla_status mla_quantize_fp8_sat(const float* src_dev, uint8_t* dst_dev, int64_t n, float scale,
                                void* stream) {
  if (n < 0 || !good_scale(scale)) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  if (src_dev == nullptr || dst_dev == nullptr) return MLA_ERR_INVALID_ARG;
  const hipError_t e = mla::launch_quantize(src_dev, dst_dev, n, scale, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_quantize_fp8_sat_dynamic(const void* src_dev, int src_dtype, uint8_t* dst_dev,
                                        int64_t n, float* scale_dev, void* workspace_dev,
                                        int64_t workspace_bytes, void* stream) {
  if (n < 0 || (src_dtype != MLA_SRC_F32 && src_dtype != MLA_SRC_BF16)) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  if (!src_dev || !dst_dev || !scale_dev || !workspace_dev) return MLA_ERR_INVALID_ARG;
  if (((uintptr_t)workspace_dev & 3) != 0 || ((uintptr_t)scale_dev & 3) != 0 ||
      ((uintptr_t)src_dev & (src_dtype == MLA_SRC_BF16 ? 1 : 3)) != 0)
    return MLA_ERR_INVALID_ARG;
  if (workspace_bytes < mla::dynamic_quantize_workspace_bytes()) return MLA_ERR_WORKSPACE;
  const hipError_t e = mla::launch_quantize_dynamic(src_dev, src_dtype == MLA_SRC_BF16, dst_dev,
                                                    n, scale_dev, workspace_dev,
                                                    (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"

namespace {

mla_status append_common(const void* new_kv_dev, int src_dtype, uint8_t* kv_pool_dev,
                         int64_t num_pages, const int32_t* page_table_dev,
                         const int32_t* seq_lens_dev, int batch, int new_tokens, int page_size,
                         int max_pages, float kv_scale, const float* rope_cos_dev,
                         const float* rope_sin_dev, int64_t rope_positions, void* stream) {
  if (batch < 0 || new_tokens < 0 || page_size < 1 || max_pages < 1 || num_pages < 1 ||
      !good_scale(kv_scale) || (src_dtype != MLA_SRC_F32 && src_dtype != MLA_SRC_BF16))
    return MLA_ERR_INVALID_ARG;
  if (batch == 0 || new_tokens == 0) return MLA_OK;
  if (!new_kv_dev || !kv_pool_dev || !page_table_dev || !seq_lens_dev) return MLA_ERR_INVALID_ARG;
  if (((uintptr_t)new_kv_dev & (src_dtype == MLA_SRC_BF16 ? 1 : 3)) != 0)
    return MLA_ERR_INVALID_ARG;
  if ((int64_t)batch * new_tokens > 0x7FFFFFFFLL ||
      (int64_t)max_pages * page_size > 0x7FFFFFFFLL)
    return MLA_ERR_UNSUPPORTED;
  const hipError_t e = mla::launch_kv_append(new_kv_dev, src_dtype == MLA_SRC_BF16, kv_pool_dev,
                                             num_pages, page_table_dev,
                                             seq_lens_dev, batch, new_tokens, page_size,
                                             max_pages, kv_scale, rope_cos_dev, rope_sin_dev,
                                             rope_positions, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

mla_status mla_kv_append_fp8_sat(const void* new_kv_dev, int src_dtype, uint8_t* kv_pool_dev,
                                 int64_t num_pages, const int32_t* page_table_dev,
                                 const int32_t* seq_lens_dev, int batch, int new_tokens,
                                 int page_size, int max_pages, float kv_scale, void* stream) {
  return append_common(new_kv_dev, src_dtype, kv_pool_dev, num_pages, page_table_dev,
                       seq_lens_dev, batch, new_tokens, page_size, max_pages, kv_scale, nullptr,
                       nullptr, 0, stream);
}

mla_status mla_kv_append_rope_fp8_sat(const void* new_kv_dev, int src_dtype, uint8_t* kv_pool_dev,
                                      int64_t num_pages, const int32_t* page_table_dev,
                                      const int32_t* seq_lens_dev, int batch, int new_tokens,
                                      int page_size, int max_pages, float kv_scale,
                                      const float* rope_cos_dev, const float* rope_sin_dev,
                                      int64_t rope_positions, void* stream) {
  if (rope_positions < 1 || rope_positions > (int64_t(1) << 40)) return MLA_ERR_INVALID_ARG;
  if (batch > 0 && new_tokens > 0 &&
      (!rope_cos_dev || !rope_sin_dev || ((uintptr_t)rope_cos_dev & 3) != 0 ||
       ((uintptr_t)rope_sin_dev & 3) != 0))
    return MLA_ERR_INVALID_ARG;
  return append_common(new_kv_dev, src_dtype, kv_pool_dev, num_pages, page_table_dev,
                       seq_lens_dev, batch, new_tokens, page_size, max_pages, kv_scale,
                       rope_cos_dev, rope_sin_dev, rope_positions, stream);
}

mla_status mla_splitkv_plan(int batch, int q_tokens, int heads, int max_seq_len,
                            int64_t total_kv_tokens, int cu_count, int* num_splits,
                            int* rows_per_group, int64_t* partial_rows) {
  if (batch < 1 || q_tokens < 1 || heads < 1 || max_seq_len < 1 || cu_count < 0 ||
      total_kv_tokens < 0 || total_kv_tokens > (int64_t)batch * max_seq_len)
    return MLA_ERR_INVALID_ARG;
  if ((int64_t)q_tokens * heads > mla::kMaxRows) return MLA_ERR_UNSUPPORTED;
  int cu = cu_count;
  if (cu == 0) {
    const mla_status st = device_cu_count(&cu);
    if (st != MLA_OK) return st;
  }
  int s = 1, r = 128;
  plan(batch, q_tokens, heads, max_seq_len, total_kv_tokens, cu, &s, &r);
  if (num_splits) *num_splits = s;
  if (rows_per_group) *rows_per_group = r;
  if (partial_rows) *partial_rows = (int64_t)batch * s * q_tokens * heads;
  return MLA_OK;
}

}  // extern "C"

namespace mla {

mla_status decode_check_args(const uint8_t* q8_dev, const uint8_t* kv_pool_dev,
                             const int32_t* page_table_dev, const int32_t* seq_lens_dev,
                             const int32_t* q_lens_dev, const int32_t* ctx_after_dev,
                             const int32_t* order_dev, int batch, int q_tokens, int heads,
                             int page_size, int max_pages, int max_seq_len, float q_scale,
                             float kv_scale, const float* q_scale_dev,
                             const float* kv_scale_dev, float softmax_scale, int num_splits,
                             int rows_per_group) {
  const bool dev = q_scale_dev != nullptr;
  if (batch < 0 || q_tokens < 1 || heads < 1 || page_size < 1 || max_pages < 1 ||
      num_splits < 0 || rows_per_group < 0)
    return MLA_ERR_INVALID_ARG;
  if ((!dev && (!good_scale(q_scale) || !good_scale(kv_scale))) || !good_scale(softmax_scale))
    return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!q8_dev || !kv_pool_dev || !page_table_dev || !seq_lens_dev) return MLA_ERR_INVALID_ARG;
  if (dev && (kv_scale_dev == nullptr || ((uintptr_t)q_scale_dev & 3) != 0 ||
              ((uintptr_t)kv_scale_dev & 3) != 0))
    return MLA_ERR_INVALID_ARG;
  if (((uintptr_t)q_lens_dev & 3) != 0 || ((uintptr_t)ctx_after_dev & 3) != 0 ||
      ((uintptr_t)order_dev & 3) != 0)
    return MLA_ERR_INVALID_ARG;
  const int64_t M = (int64_t)q_tokens * heads;
  if (M > kMaxRows || page_size % kTile != 0 ||
      (int64_t)max_pages * page_size + 2LL * q_tokens > 0x7FFFFFFFLL - 64)
    return MLA_ERR_UNSUPPORTED;
  if (rows_per_group != 0 && rows_per_group != 128) return MLA_ERR_UNSUPPORTED;
  if ((num_splits == 0 || rows_per_group == 0) && max_seq_len < 1) return MLA_ERR_INVALID_ARG;
  if (num_splits > 65535) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

}  // namespace mla

namespace {

// Every decode entry point: host scales (q_scale_dev == NULL) or device scales; one query
// count for all requests (q_lens_dev == NULL) or one per request.
mla_status decode_common(const uint8_t* q8_dev, const uint8_t* kv_pool_dev,
                         const int32_t* page_table_dev, const int32_t* seq_lens_dev,
                         const int32_t* q_lens_dev, const int32_t* ctx_after_dev,
                         const int32_t* order_dev, int batch,
                         int q_tokens, int heads, int page_size, int max_pages, int max_seq_len,
                         float q_scale, float kv_scale, const float* q_scale_dev,
                         const float* kv_scale_dev, float softmax_scale, int num_splits,
                         int rows_per_group, uint16_t* partial_o_dev, float* partial_lse_dev,
                         int64_t partial_rows_capacity, void* stream) {
  if (partial_rows_capacity < 0) return MLA_ERR_INVALID_ARG;
  const mla_status chk = mla::decode_check_args(
      q8_dev, kv_pool_dev, page_table_dev, seq_lens_dev, q_lens_dev, ctx_after_dev, order_dev,
      batch, q_tokens, heads, page_size, max_pages, max_seq_len, q_scale, kv_scale, q_scale_dev,
      kv_scale_dev, softmax_scale, num_splits, rows_per_group);
  if (chk != MLA_OK || batch == 0) return chk;
  if (!partial_o_dev || !partial_lse_dev) return MLA_ERR_INVALID_ARG;
  const int64_t M = (int64_t)q_tokens * heads;
  int S = num_splits, r = rows_per_group;
  if (S == 0 || r == 0) {
    int cu = 0;
    const mla_status st = device_cu_count(&cu);
    if (st != MLA_OK) return st;
    int ps = 1, pr = 128;
    plan(batch, q_tokens, heads, max_seq_len, 0, cu, &ps, &pr);
    if (S == 0) S = ps;
    if (r == 0) r = pr;
  }
  if (S > 65535) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)batch * S * M > partial_rows_capacity) return MLA_ERR_WORKSPACE;
  const int64_t groups = cdiv(M, r);
  if (cdiv((int64_t)batch * S, 8) * 8 * groups > 0x7FFFFFFFLL) return MLA_ERR_UNSUPPORTED;

  mla::DecodeParams p;
  p.q8 = q8_dev;
  p.kv = kv_pool_dev;
  p.page_table = page_table_dev;
  p.seq_lens = seq_lens_dev;
  p.partial_o = partial_o_dev;
  p.partial_lse = partial_lse_dev;
  p.batch = batch;
  p.q_tokens = q_tokens;
  p.heads = heads;
  p.rows = (int)M;
  p.page_size = page_size;
  p.page_bytes = (int64_t)page_size * mla::kD;
  {  // prefetch hint only (any value is safe): a split's tiles if every length were the maximum
    const int64_t ms = max_seq_len < 1 ? 1 : max_seq_len;
    const int64_t tiles = cdiv(ms, (int64_t)mla::kTile);
    const int64_t per = 2 * cdiv(cdiv(tiles, 2), (int64_t)S);  // whole 64-token steps
    p.tiles_hint = (int)(per > 0x7FFF ? 0x7FFF : per);
  }
  p.max_pages = max_pages;
  p.num_splits = S;
  p.groups = (int)groups;
  p.div_splits = mla::make_fastdiv((uint32_t)S);
  p.div_groups = mla::make_fastdiv((uint32_t)groups);
  p.div_heads = mla::make_fastdiv((uint32_t)heads);
  p.div_tpp = mla::make_fastdiv((uint32_t)(page_size / mla::kTile));
  p.c2 = q_scale_dev != nullptr ? 0.f : mla::score_scale_log2(q_scale, kv_scale, softmax_scale);
  p.kv_scale = kv_scale;
  p.q_scale_dev = q_scale_dev;
  p.kv_scale_dev = kv_scale_dev;
  p.softmax_scale = softmax_scale;
  p.q_lens = q_lens_dev;
  p.ctx_after = ctx_after_dev;
  p.order = order_dev;
  const hipError_t e = mla::launch_decode(p, r, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status combine_common(const uint16_t* partial_o_dev, const float* partial_lse_dev,
                          int batch, int num_splits, int q_tokens, int heads, float v_scale,
                          const float* v_scale_dev, uint16_t* out_bf16_dev, float* out_lse_dev,
                          void* stream) {
  if (batch < 0 || num_splits < 1 || q_tokens < 1 || heads < 1) return MLA_ERR_INVALID_ARG;
  if (v_scale_dev == nullptr && !good_scale(v_scale)) return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!partial_o_dev || !partial_lse_dev || !out_bf16_dev) return MLA_ERR_INVALID_ARG;
  if (((uintptr_t)v_scale_dev & 3) != 0) return MLA_ERR_INVALID_ARG;
  const int64_t M = (int64_t)q_tokens * heads;
  if (M > mla::kMaxRows || num_splits > mla::kMaxSplitsCombine) return MLA_ERR_UNSUPPORTED;
  if ((int64_t)batch * M * 2 > 0x7FFFFFFFLL) return MLA_ERR_UNSUPPORTED;
  const hipError_t e = mla::launch_combine(partial_o_dev, partial_lse_dev, batch, num_splits,
                                           (int)M, v_scale, v_scale_dev, out_bf16_dev,
                                           out_lse_dev, M, false, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

mla_status mla_decode_splitkv(const uint8_t* q8_dev, const uint8_t* kv_pool_dev,
                              const int32_t* page_table_dev, const int32_t* seq_lens_dev,
                              int batch, int q_tokens, int heads, int page_size, int max_pages,
                              int max_seq_len, float q_scale, float kv_scale, float softmax_scale,
                              int num_splits, int rows_per_group, uint16_t* partial_o_dev,
                              float* partial_lse_dev, int64_t partial_rows_capacity,
                              void* stream) {
  return decode_common(q8_dev, kv_pool_dev, page_table_dev, seq_lens_dev, nullptr, nullptr,
                       nullptr, batch,
                       q_tokens, heads, page_size, max_pages, max_seq_len, q_scale, kv_scale,
                       nullptr, nullptr,
                       softmax_scale, num_splits, rows_per_group, partial_o_dev, partial_lse_dev,
                       partial_rows_capacity, stream);
}

mla_status mla_decode_splitkv_dev_scales(const uint8_t* q8_dev, const uint8_t* kv_pool_dev,
                                         const int32_t* page_table_dev,
                                         const int32_t* seq_lens_dev, int batch, int q_tokens,
                                         int heads, int page_size, int max_pages,
                                         int max_seq_len, const float* q_scale_dev,
                                         const float* kv_scale_dev, float softmax_scale,
                                         int num_splits, int rows_per_group,
                                         uint16_t* partial_o_dev, float* partial_lse_dev,
                                         int64_t partial_rows_capacity, void* stream) {
  if (q_scale_dev == nullptr || kv_scale_dev == nullptr) return MLA_ERR_INVALID_ARG;
  return decode_common(q8_dev, kv_pool_dev, page_table_dev, seq_lens_dev, nullptr, nullptr,
                       nullptr, batch,
                       q_tokens, heads, page_size, max_pages, max_seq_len, 1.0f, 1.0f,
                       q_scale_dev, kv_scale_dev,
                       softmax_scale, num_splits, rows_per_group, partial_o_dev, partial_lse_dev,
                       partial_rows_capacity, stream);
}

mla_status mla_decode_splitkv_ex(const uint8_t* q8_dev, const uint8_t* kv_pool_dev,
                                 const int32_t* page_table_dev, const int32_t* seq_lens_dev,
                                 const int32_t* q_lens_dev, const int32_t* ctx_after_dev,
                                 const int32_t* order_dev, int batch, int q_tokens, int heads,
                                 int page_size, int max_pages, int max_seq_len, float q_scale,
                                 float kv_scale, const float* q_scale_dev,
                                 const float* kv_scale_dev, float softmax_scale, int num_splits,
                                 int rows_per_group, uint16_t* partial_o_dev,
                                 float* partial_lse_dev, int64_t partial_rows_capacity,
                                 void* stream) {
  if ((q_scale_dev == nullptr) != (kv_scale_dev == nullptr)) return MLA_ERR_INVALID_ARG;
  return decode_common(q8_dev, kv_pool_dev, page_table_dev, seq_lens_dev, q_lens_dev,
                       ctx_after_dev, order_dev, batch,
                       q_tokens, heads, page_size, max_pages, max_seq_len, q_scale, kv_scale,
                       q_scale_dev, kv_scale_dev, softmax_scale, num_splits, rows_per_group,
                       partial_o_dev, partial_lse_dev, partial_rows_capacity, stream);
}

mla_status mla_splitkv_combine(const uint16_t* partial_o_dev, const float* partial_lse_dev,
                               int batch, int num_splits, int q_tokens, int heads, float v_scale,
                               uint16_t* out_bf16_dev, float* out_lse_dev, void* stream) {
  return combine_common(partial_o_dev, partial_lse_dev, batch, num_splits, q_tokens, heads,
                        v_scale, nullptr, out_bf16_dev, out_lse_dev, stream);
}

mla_status mla_splitkv_combine_partial(const uint16_t* partial_o_dev,
                                       const float* partial_lse_dev, int batch, int num_splits,
                                       int q_tokens, int heads, uint16_t* out_partial_o_dev,
                                       float* out_partial_lse_dev, int64_t out_batch_stride_rows,
                                       void* stream) {
  if (batch < 0 || num_splits < 1 || q_tokens < 1 || heads < 1) return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!partial_o_dev || !partial_lse_dev || !out_partial_o_dev || !out_partial_lse_dev)
    return MLA_ERR_INVALID_ARG;
  const int64_t M = (int64_t)q_tokens * heads;
  if (M > mla::kMaxRows || num_splits > mla::kMaxSplitsCombine) return MLA_ERR_UNSUPPORTED;
  if (out_batch_stride_rows < M) return MLA_ERR_INVALID_ARG;
  if ((int64_t)batch * M * 2 > 0x7FFFFFFFLL) return MLA_ERR_UNSUPPORTED;
  const hipError_t e = mla::launch_combine(partial_o_dev, partial_lse_dev, batch, num_splits,
                                           (int)M, 1.0f, nullptr, out_partial_o_dev,
                                           out_partial_lse_dev, out_batch_stride_rows, true,
                                           (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status mla_splitkv_combine_dev_scale(const uint16_t* partial_o_dev,
                                         const float* partial_lse_dev, int batch,
                                         int num_splits, int q_tokens, int heads,
                                         const float* v_scale_dev, uint16_t* out_bf16_dev,
                                         float* out_lse_dev, void* stream) {
  if (v_scale_dev == nullptr) return MLA_ERR_INVALID_ARG;
  return combine_common(partial_o_dev, partial_lse_dev, batch, num_splits, q_tokens, heads, 1.0f,
                        v_scale_dev, out_bf16_dev, out_lse_dev, stream);
}

mla_status mla_hbm_read_probe(const void* buf_dev, int64_t bytes, uint32_t* out_dev,
                              int grid, void* stream) {
  if (buf_dev == nullptr || out_dev == nullptr || grid < 1 || bytes < 0 ||
      bytes % mla::read_probe_chunk_bytes() != 0 || ((uintptr_t)buf_dev & 15) != 0)
    return MLA_ERR_INVALID_ARG;
  if (bytes == 0) return MLA_OK;
  const hipError_t e = mla::launch_read_probe(buf_dev, bytes, out_dev, grid, (hipStream_t)stream);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
