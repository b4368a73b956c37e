/*
 * mla.h -- C ABI of libmla.so: FP8 MLA split-KV decode for AMD Instinct MI355X (gfx950).
 *
 * Sources cited below:
 *   [A]      the arex-research.com page "SGLang 与 Miles 团队称在预发布 Vera Rubin 上跑通
 *            Kimi K3 推理和端到端 RL，自测 FP8 MLA 提速最高约 20%".
 *   [A/MLA]  its section "Kimi K3 的 MLA：更深的流水线、更快的 split-KV 归约"; the section's
 *            list has four items: (1) deeper MLA pipeline, (2) faster split-KV reduction,
 *            (3) 64-way split-KV, (4) native saturating FP8 conversion.
 *   [B]      the ai.newsbites.today page "LMSYS、NVIDIA Rubin向けの高速化成果を発表", section
 *            "MLAアテンションのパイプライン深化".
 *   [C]      the theainews.cc page on Muse Spark Open, section "内核优化:解码吞吐 3 倍", item
 *            "RoPE 与 KV 缓存写入融合" (RoPE applied in the kernel that writes the decode KV).
 *
 * Problem (the pages' statement, in our words): long-context MLA decode mostly waits on
 * reading the KV cache from HBM ([A/MLA] (1), [B]).  Q and KV are first converted to FP8
 * with a saturating cast ([A/MLA] (4)); at low batch one request's KV is split over many
 * workgroups, each producing a partial result, and a second kernel merges the partials
 * ([A/MLA] (2), (3)).  The KV row is 576 bytes wide (512 latent + 64 rope columns, shared
 * by all query heads); the value vector is the row's first 512 columns.
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev are device pointers (HIP device memory); everything else is
 *     passed by value.  The caller allocates and frees every buffer; the library never
 *     allocates, frees or synchronises.  Its state is a per-device cache of the compute-unit
 *     count, filled on first use, and, for mla_decode_noalloc only, one device array per GPU
 *     (part of the library's code object, not allocated at run time) whose address it looks
 *     up on that GPU's first such call.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.  Work is
 *     enqueued asynchronously; device-side faults surface at the caller's next sync.
 *   - Every argument check runs before any HIP call, so invalid arguments are reported
 *     on a host without a GPU.  Nothing throws across the ABI and nothing aborts.
 *   - FP8 here is OCP E4M3 without infinities (max 448, NaN = S.1111.111), the format
 *     gfx950's conversion and matrix instructions use.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1, /* null pointer where one is required, negative size, non-finite
                              or non-positive scale */
  MLA_ERR_UNSUPPORTED = 2, /* well-formed but outside the supported shapes (see each call) */
  MLA_ERR_WORKSPACE = 3,   /* partial buffers too small for the requested split count */
  MLA_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  /* Not statuses: these two bounds make every int a value of the type, so a code from
     anywhere (an older or newer library, a corrupted variable) can be passed to
     mla_status_string without undefined behaviour in C++. */
  MLA_STATUS_INT_MIN_ = -2147483647 - 1,
  MLA_STATUS_INT_MAX_ = 2147483647
} mla_status;

/* Human-readable name of a status code; "MLA_ERR_UNKNOWN" for any other int (static
   storage, never NULL). */
const char* mla_status_string(mla_status s);

/*
 * Saturating FP8 quantisation of a contiguous fp32 array ([A/MLA] item (4)).
 *
 *   dst_dev[i] = e4m3_sat_rne(float32(src_dev[i]) / scale)   for i in [0, n)
 *
 * The quotient is an IEEE fp32 division.  It is rounded to the nearest E4M3 value, ties to
 * the even code.  Every finite |quotient| >= 448 and +-inf saturate to 0x7E | sign (never
 * NaN); NaN becomes 0x7F | sign; the sign of zero is kept.  With a per-tensor scale
 * amax / 448 the largest magnitude maps to 448.
 *   src_dev : fp32 [n], device.        dst_dev : uint8 [n], device (may not alias src_dev).
 *   n       : element count, >= 0 (0 enqueues nothing).
 *   scale   : finite, > 0.
 * Errors: INVALID_ARG for n < 0, a NULL pointer with n > 0, or a bad scale; HIP on launch
 * failure.
 */
mla_status mla_quantize_fp8_sat(const float* src_dev, uint8_t* dst_dev, int64_t n, float scale,
                                void* stream);

/*
 * Saturating FP8 quantisation with the per-tensor scale taken from the data on the device
 * ([A/MLA] item (4); the scale is the usual amax / 448, so the caller needs no host copy of
 * the tensor's range and no synchronisation before the decode):
 *
 *   x_i       = src_dev[i] as fp32 (a bf16 source is widened exactly: its bits are the upper
 *               half of the fp32 pattern)
 *   amax      = max_i |x_i|
 *   scale     = 1 if amax == 0, else float32(amax) / 448 (IEEE fp32 division)
 *   dst_dev[i] = the code of mla_quantize_fp8_sat for x_i with that scale
 *   scale_dev[0] = scale
 *
 * A tensor holding a NaN gets a NaN scale (and NaN codes); one holding +-inf an inf scale.
 *   src_dev   : device, fp32 [n] (src_dtype MLA_SRC_F32, 4-byte aligned) or bf16 bit
 *               patterns [n] (MLA_SRC_BF16, 2-byte aligned).
 *   dst_dev   : uint8 [n], device (may not alias src_dev).   n >= 0 (0 enqueues nothing).
 *   scale_dev : one float, device, 4-byte aligned; written by the second of the two kernels
 *               this call enqueues (the first writes per-workgroup maxima to the workspace).
 *   workspace_dev / workspace_bytes : device scratch, 4-byte aligned, at least
 *               MLA_QUANTIZE_DYNAMIC_WORKSPACE_BYTES; its contents on entry do not matter.
 *               Calls that share a workspace must not run concurrently.
 * Errors: INVALID_ARG (n < 0, unknown dtype, NULL or misaligned pointers with n > 0);
 * WORKSPACE (workspace too small); HIP.
 */
#define MLA_QUANTIZE_DYNAMIC_WORKSPACE_BYTES 4096
enum { MLA_SRC_F32 = 0, MLA_SRC_BF16 = 1 };
mla_status mla_quantize_fp8_sat_dynamic(const void* src_dev, int src_dtype, uint8_t* dst_dev,
                                        int64_t n, float* scale_dev, void* workspace_dev,
                                        int64_t workspace_bytes, void* stream);

/*
 * Append a decode step's new latent + rope rows to the paged FP8 KV cache, quantised on the
 * way in ([A/MLA] item (4): KV is converted to FP8 before the attention reads it; here the
 * conversion writes straight into the cache the decode call reads).
 *
 * New token t (0 <= t < T) of request b is logical position n = seq_lens_dev[b] - T + t, i.e.
 * seq_lens_dev already counts the T new tokens, as mla_decode_splitkv expects.  Its row
 *   kv_pool[page_table[b, n / page_size], n % page_size, 0:576]
 *     = e4m3_sat_rne(float32(new_kv[b, t, :]) / kv_scale)      (as mla_quantize_fp8_sat)
 * Positions outside [0, max_pages * page_size) and page ids outside [0, num_pages) are not
 * written; no other byte of the pool changes.  If two new rows name the same cache row,
 * which one lands is unspecified.
 *   new_kv_dev     [B, T, 576], device: fp32 (src_dtype MLA_SRC_F32, 4-byte aligned) or
 *                  bf16 bit patterns (MLA_SRC_BF16, 2-byte aligned; widened exactly to fp32
 *                  before the division); 16-byte alignment of it and of the pool takes the
 *                  vector path; may not alias the pool.
 *   kv_pool_dev    uint8 [num_pages, page_size, 576], device.
 *   page_table_dev int32 [B, max_pages];  seq_lens_dev int32 [B]  (device).
 *   kv_scale       the cache's dequantisation scale: finite, > 0.
 * Errors: INVALID_ARG (negative sizes, page_size/max_pages/num_pages < 1, bad scale, unknown
 * src_dtype, NULL or misaligned pointers with B*T > 0); UNSUPPORTED (B*T or
 * max_pages*page_size >= 2^31); HIP.
 * B == 0 or T == 0 enqueues nothing.
 */
mla_status mla_kv_append_fp8_sat(const void* new_kv_dev, int src_dtype, uint8_t* kv_pool_dev,
                                 int64_t num_pages, const int32_t* page_table_dev,
                                 const int32_t* seq_lens_dev, int batch, int new_tokens,
                                 int page_size, int max_pages, float kv_scale, void* stream);

/*
 * mla_kv_append_fp8_sat with the rotary position embedding applied on the way in ([C]: RoPE
 * fused with the KV-cache write, so no separate kernel rotates the new rows first).  The new
 * rows carry the rope part unrotated; for new token t of request b at position
 * n = seq_lens_dev[b] - T + t, the 32 pairs of adjacent rope columns (512 + 2i, 513 + 2i) are
 * rotated as complex numbers by the angle of pair i at position n:
 *   r0 = fl(fl(x0 * c) - fl(x1 * s)),   r1 = fl(fl(x0 * s) + fl(x1 * c)),
 *   c = rope_cos_dev[n * 32 + i],  s = rope_sin_dev[n * 32 + i]
 * in fp32 with every product and sum rounded on its own (no fused multiply-add), then the whole
 * 576-wide row is quantised and stored exactly as mla_kv_append_fp8_sat does (the 512 latent
 * columns are not rotated).  A position n >= rope_positions is not written (as a position past
 * the page table).
 *   rope_cos_dev, rope_sin_dev : fp32 [rope_positions, 32], device, 4-byte aligned (16-byte
 *                                aligned ones take the vector path): the caller's angle tables,
 *                                so any frequency schedule can be used.
 *   rope_positions            : rows of the tables, >= 1.
 * Other arguments, conventions and errors as mla_kv_append_fp8_sat, plus INVALID_ARG for
 * NULL or misaligned tables (with B*T > 0) and rope_positions < 1.
 */
mla_status mla_kv_append_rope_fp8_sat(const void* new_kv_dev, int src_dtype, uint8_t* kv_pool_dev,
                                      int64_t num_pages, const int32_t* page_table_dev,
                                      const int32_t* seq_lens_dev, int batch, int new_tokens,
                                      int page_size, int max_pages, float kv_scale,
                                      const float* rope_cos_dev, const float* rope_sin_dev,
                                      int64_t rope_positions, void* stream);

/*
 * Split planner ([A/MLA] item (3): at batch 1 a fixed split count leaves most compute units
 * idle; the count has to follow the machine and the shape).  Chooses, from the compute-unit
 * count, the batch, the number of query rows (q_tokens * heads) and the longest context:
 *   *num_splits      S, the number of KV chunks per request (>= 1);
 *   *rows_per_group  query rows handled by one workgroup (128).  Rows are the
 *                    (query token, head) pairs of a request in [Sq, H] order; a request's
 *                    rows are covered by ceil(Sq*H / rows_per_group) workgroups per chunk,
 *                    which read the chunk's KV through the same L2;
 *   *partial_rows    B * S * Sq * H: the entries mla_decode_splitkv writes, i.e. the sizes
 *                    of partial_o (x 512 fp16 values) and partial_lse (x 1 float).
 *   total_kv_tokens : the sum of the requests' lengths when the caller knows it (mixed
 *                    lengths: the split count then balances the total work over the CUs
 *                    against the longest request's chunks); 0 = every request is
 *                    max_seq_len long (what mla_decode_splitkv assumes when it plans);
 *   cu_count : compute units to plan for; 0 queries the current device (a HIP call).
 * Any output pointer may be NULL.  Errors: INVALID_ARG for batch, q_tokens, heads or
 * max_seq_len < 1, cu_count < 0, or total_kv_tokens outside [0, batch * max_seq_len];
 * UNSUPPORTED when q_tokens * heads > 65536.
 */
mla_status mla_splitkv_plan(int batch, int q_tokens, int heads, int max_seq_len,
                            int64_t total_kv_tokens, int cu_count, int* num_splits,
                            int* rows_per_group, int64_t* partial_rows);

/*
 * Split-KV partial attention over an FP8 paged KV cache ([A/MLA] items (1)-(3), [B]).
 *
 * For request b, query token t and head h (row r = t * H + h), and for chunk s of the
 * request's tokens, computes over the positions n of that chunk that the row may see
 * (bottom-right causal: n <= L_b - Sq + t, with L_b = seq_lens_dev[b] counting the Sq query
 * tokens):
 *   z_n  = softmax_scale * q_scale * kv_scale * (dec(Q8[b,t,h,:]) . dec(KV8[n,:]))
 *   partial_lse[b,s,r]    = log(sum_n exp(z_n))          (natural log; -inf if no position)
 *   partial_o[b,s,r,0:512] = sum_n softmax(z)_n * dec(KV8[n,0:512])
 * i.e. the chunk's attention output in units of kv_scale, so every value lies in [-448, 448]
 * and is stored as IEEE fp16 (round to nearest even); mla_splitkv_combine multiplies by
 * kv_scale again.  Chunk s holds tiles [s*c, (s+1)*c) of 32 tokens, c = 2 * ceil(ceil(L_b/64)
 * / S), i.e. whole 64-token steps (the last chunks of a short request may be empty).  Where
 * the lse is -inf (empty chunk, or no visible position) the partial_o entry is unspecified.
 *
 * Layouts (all contiguous, row-major):
 *   q8_dev          uint8 [B, Sq, H, 576]          e4m3 codes of Q
 *   kv_pool_dev     uint8 [num_pages, page_size, 576]  e4m3 codes of the latent+rope KV
 *   page_table_dev  int32 [B, max_pages]   logical token n of request b is row n % page_size
 *                                          of page page_table[b, n / page_size]
 *   seq_lens_dev    int32 [B]              context length per request (device values are
 *                                          clamped to [0, max_pages * page_size])
 *   partial_o_dev   fp16 bits [B, S, Sq*H, 512];  partial_lse_dev fp32 [B, S, Sq*H]
 * A contiguous per-request cache is the same call with page_size = the padded length and
 * page_table[b] = {b}.
 *   max_seq_len   : host upper bound of the lengths, used only when num_splits == 0.
 *   num_splits    : S >= 1, or 0 to take the planner's choice for (B, Sq, H, max_seq_len).
 *   rows_per_group: 128, or 0 to take the planner's choice.
 *   partial_rows_capacity : entries the partial buffers hold (see mla_splitkv_plan).
 * Supported: 1 <= Sq, Sq*H <= 65536, page_size a positive multiple of 32, max_pages >= 1,
 * max_pages * page_size + 2 * Sq < 2^31 - 64, num_splits <= 65535 (mla_splitkv_combine
 * merges at most 4096 in one call; the planner never picks more).
 * Errors: INVALID_ARG (NULL pointers with B > 0, negative sizes, scales not finite and > 0);
 * UNSUPPORTED (shape outside the supported set); WORKSPACE (B*S*Sq*H > capacity); HIP.
 * B == 0 enqueues nothing.
 */
mla_status mla_decode_splitkv(const uint8_t* q8_dev, const uint8_t* kv_pool_dev,
                              const int32_t* page_table_dev, const int32_t* seq_lens_dev,
                              int batch, int q_tokens, int heads, int page_size, int max_pages,
                              int max_seq_len, float q_scale, float kv_scale, float softmax_scale,
                              int num_splits, int rows_per_group,
                              uint16_t* partial_o_dev, float* partial_lse_dev,
                              int64_t partial_rows_capacity, void* stream);

/*
 * mla_decode_splitkv with both dequantisation scales read on the device: q_scale_dev[0] and
 * kv_scale_dev[0] (4-byte aligned device floats, e.g. written by
 * mla_quantize_fp8_sat_dynamic earlier on the same stream) take the place of q_scale and
 * kv_scale, so a step whose Q scale comes from the data needs no host round trip
 * ([A/MLA] item (4) with a data-derived scale).  The kernel forms the score factor from them
 * exactly as the host does (products in double, one rounding to float), so equal scale
 * values give bit-identical partials.  The scales must be finite and > 0 (not checked: they
 * live on the device).  Errors as mla_decode_splitkv, plus INVALID_ARG for a NULL or
 * misaligned scale pointer.
 */
mla_status mla_decode_splitkv_dev_scales(const uint8_t* q8_dev, const uint8_t* kv_pool_dev,
                                         const int32_t* page_table_dev,
                                         const int32_t* seq_lens_dev, int batch, int q_tokens,
                                         int heads, int page_size, int max_pages,
                                         int max_seq_len, const float* q_scale_dev,
                                         const float* kv_scale_dev, float softmax_scale,
                                         int num_splits, int rows_per_group,
                                         uint16_t* partial_o_dev, float* partial_lse_dev,
                                         int64_t partial_rows_capacity, void* stream);

/*
 * The general form of the decode call: mla_decode_splitkv plus
 *   q_lens_dev   int32 [B] (device) or NULL.  Request b has q_lens_dev[b] query tokens
 *                (device values are clamped to [0, q_tokens]): the verify step of block
 *                speculative decoding ([A/MLA], opening paragraph: every decode step drafts a
 *                few tokens, then verifies them) with a different number of draft tokens per
 *                request.  Its tokens are the
 *                first q_lens_dev[b] of the q_tokens slots of q8 and are the last
 *                q_lens_dev[b] positions of its context: token t sees positions
 *                0 .. L_b - q_lens_dev[b] + t.  Rows of slots t >= q_lens_dev[b] see nothing:
 *                their partial lse is -inf in every split, so the combine gives O = 0 and
 *                lse = -inf for them.  NULL: every request has q_tokens tokens.
 *   ctx_after_dev int32 [B] (device) or NULL.  The number of request b's context positions
 *                that come after the L_b positions this call reads (device values clamped to
 *                [0, q_tokens]; 0 = none).  For a request whose KV is split into
 *                contiguous shards (on several GPUs, say): the query tokens are the last
 *                positions of the whole context, so position n of this shard is visible to
 *                token t when n <= L_b + ctx_after[b] - q_lens[b] + t; with ctx_after[b] >=
 *                q_lens[b] every position of the shard is visible.  Each shard's partials
 *                (merged by mla_splitkv_combine_partial) then combine into the request's
 *                output.  NULL: the call sees the end of every request's context.
 *   order_dev    int32 [B] (device) or NULL.  A permutation of the requests: the workgroups
 *                of request order_dev[0] are dispatched first, then those of order_dev[1],
 *                and so on.  Every request's chunk size follows its own length, so when
 *                lengths differ, putting the longest requests first (the caller knows the
 *                lengths) keeps the last-dispatched workgroups short and the CUs evenly
 *                loaded.  The result does not depend on it.  Values are clamped into
 *                [0, B); an order that is not a permutation computes some requests twice
 *                and leaves others unwritten.  NULL: request order.
 *   q_scale_dev, kv_scale_dev  both NULL (q_scale and kv_scale are used) or both device
 *                floats (as mla_decode_splitkv_dev_scales).
 * Errors as mla_decode_splitkv, plus INVALID_ARG for exactly one NULL scale pointer or a
 * misaligned pointer.
 */
mla_status mla_decode_splitkv_ex(const uint8_t* q8_dev, const uint8_t* kv_pool_dev,
                                 const int32_t* page_table_dev, const int32_t* seq_lens_dev,
                                 const int32_t* q_lens_dev, const int32_t* ctx_after_dev,
                                 const int32_t* order_dev, int batch, int q_tokens, int heads,
                                 int page_size, int max_pages, int max_seq_len, float q_scale,
                                 float kv_scale, const float* q_scale_dev,
                                 const float* kv_scale_dev, float softmax_scale, int num_splits,
                                 int rows_per_group, uint16_t* partial_o_dev,
                                 float* partial_lse_dev, int64_t partial_rows_capacity,
                                 void* stream);

/*
 * Log-sum-exp merge of the split partials ([A/MLA] item (2)).  For each (b, r):
 *   M = max_s lse_s;  w_s = exp(lse_s - M);  O = v_scale * sum_s w_s O_s / sum_s w_s;
 *   lse = M + log(sum_s w_s)
 * Splits with lse_s = -inf are skipped (their partial_o is never read as a weight);
 * a row whose splits are all empty gives O = 0 and lse = -inf.  Each workgroup issues all
 * of a row's partial loads before it accumulates them in registers.
 *   partial_o_dev fp16 bits [B, S, R, 512] (as mla_decode_splitkv writes them, in units of
 *                 v_scale), partial_lse_dev fp32 [B, S, R] with R = Sq * H;
 *   v_scale       the KV dequantisation scale the partials were computed with (finite, > 0);
 *   out_bf16_dev  uint16 [B, Sq, H, 512]: bf16 bit patterns, round-to-nearest-even;
 *   out_lse_dev   fp32 [B, Sq, H] or NULL.
 * Errors: INVALID_ARG (NULL inputs/outputs with B > 0, sizes < 1, bad v_scale); UNSUPPORTED
 * (S > 4096 or Sq*H > 65536); HIP.  B == 0 enqueues nothing.
 */
mla_status mla_splitkv_combine(const uint16_t* partial_o_dev, const float* partial_lse_dev,
                               int batch, int num_splits, int q_tokens, int heads, float v_scale,
                               uint16_t* out_bf16_dev, float* out_lse_dev, void* stream);

/*
 * The same log-sum-exp merge, with the result written as one partial in the format
 * mla_decode_splitkv writes (fp16 bits in units of the KV scale, natural-log lse) instead of
 * the bf16 output, so that merged results can be merged again ([A/MLA] item (2) applied in
 * two levels).  The use it is made for: a request's KV held in contiguous shards on several
 * GPUs (context parallel); each GPU decodes its shard and merges its own splits here into
 * one partial row per (b, query row), the GPUs exchange those rows (Sq*H*1028 bytes per
 * request per GPU), and mla_splitkv_combine over the G gathered partials gives the output.
 *   partial_o_dev / partial_lse_dev   as for mla_splitkv_combine ([B, S, R, 512] / [B, S, R],
 *                                      R = Sq * H);
 *   out_partial_o_dev   fp16 bits; row b * out_batch_stride_rows + r receives (b, r)'s merged
 *                       512 values;   out_partial_lse_dev  fp32, same row index;
 *   out_batch_stride_rows  >= R: R for a [B, R] result; G * R to write slice g of a
 *                       [B, G, R] buffer (pass the pointers offset by g * R rows).
 * Rows whose splits are all empty get lse = -inf (and O = 0).
 * Errors: INVALID_ARG (NULL pointers with B > 0, sizes < 1, stride < R); UNSUPPORTED
 * (S > 4096 or Sq*H > 65536); HIP.  B == 0 enqueues nothing.
 */
mla_status mla_splitkv_combine_partial(const uint16_t* partial_o_dev,
                                       const float* partial_lse_dev, int batch, int num_splits,
                                       int q_tokens, int heads, uint16_t* out_partial_o_dev,
                                       float* out_partial_lse_dev, int64_t out_batch_stride_rows,
                                       void* stream);

/*
 * mla_splitkv_combine with v_scale read on the device from v_scale_dev[0] (a 4-byte aligned
 * device float, finite and > 0; the KV scale the partials were computed with).  Output is
 * bit-identical to mla_splitkv_combine with the same value.  Errors as mla_splitkv_combine,
 * plus INVALID_ARG for a NULL or misaligned v_scale_dev.
 */
mla_status mla_splitkv_combine_dev_scale(const uint16_t* partial_o_dev,
                                         const float* partial_lse_dev, int batch,
                                         int num_splits, int q_tokens, int heads,
                                         const float* v_scale_dev, uint16_t* out_bf16_dev,
                                         float* out_lse_dev, void* stream);

/*
 * mla_decode_splitkv followed by mla_splitkv_combine, allocating nothing: for callers that
 * cannot allocate device memory (work captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc).  The caller passes the inputs and outputs; the split
 * partials go to a device array of MLA_NOALLOC_SCRATCH_BYTES that the library holds on each
 * GPU it runs on, from that GPU's first call until the process ends (its address is looked up
 * on the first call on each device; that call may load the library's code there).
 *   Inputs, scales and num_splits as for mla_decode_splitkv (rows_per_group is the planner's
 *   128); outputs as for mla_splitkv_combine: out_bf16_dev [B, Sq, H, 512] bf16 bits, out_lse_dev
 *   [B, Sq, H] fp32 or NULL.
 *   The partials need B * S * Sq * H * 1028 bytes (fp16 row + lse).  num_splits > 0 that does
 *   not fit returns MLA_ERR_WORKSPACE; num_splits == 0 takes the planner's split count,
 *   reduced until it fits (MLA_ERR_WORKSPACE if one split does not: B * Sq * H > 40,800).
 *   The result equals that of the two calls with the same split count, bit for bit.
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other host threads) race and must not be issued; calls on one stream are ordered.
 * The stream must belong to the current device (the array's address is that device's).
 * Errors: as mla_decode_splitkv and mla_splitkv_combine, plus INVALID_ARG for a NULL
 * out_bf16_dev with B > 0 or a stream of another device, WORKSPACE as above, HIP if the
 * array's address or the stream's device cannot be found.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (40 * 1024 * 1024)
mla_status mla_decode_noalloc(const uint8_t* q8_dev, const uint8_t* kv_pool_dev,
                              const int32_t* page_table_dev, const int32_t* seq_lens_dev,
                              int batch, int q_tokens, int heads, int page_size, int max_pages,
                              int max_seq_len, float q_scale, float kv_scale, float softmax_scale,
                              int num_splits, uint16_t* out_bf16_dev, float* out_lse_dev,
                              void* stream);

/*
 * Diagnostics, not part of the decode path: streams bytes of buf_dev from HBM (16-byte
 * non-temporal loads, eight in flight per lane) and writes one XOR-fold word per workgroup
 * to out_dev[0 .. grid-1].  Benchmarks time it to state the read rate the decode kernel's KV
 * traffic is compared with, on the same GPU in the same run.
 *   buf_dev  device buffer, 16-byte aligned; bytes a multiple of 32 KiB (>= 0);
 *   out_dev  uint32 [grid] (device); grid >= 1 workgroups of 256 lanes.
 * Errors: INVALID_ARG (NULL pointers, misalignment, bytes not a multiple of 32 KiB, grid < 1);
 * HIP.  bytes == 0 enqueues nothing.
 */
mla_status mla_hbm_read_probe(const void* buf_dev, int64_t bytes, uint32_t* out_dev, int grid,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
