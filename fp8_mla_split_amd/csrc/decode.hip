// Split-KV partial attention for MLA decode over an FP8 (OCP E4M3) KV cache, gfx950.
//
// Cited pages: [A] the arex-research.com Vera Rubin / Kimi K3 write-up, section "Kimi K3 的
// MLA：更深的流水线、更快的 split-KV 归约" (items: deeper pipeline, faster split-KV reduction,
// 64-way split, saturating FP8 conversion); [B] the ai.newsbites.today summary, section
// "MLAアテンションのパイプライン深化".  They state that long-context MLA decode waits mostly
// on KV reads from HBM and is made faster by keeping more reads in flight (a deeper staging
// pipeline), and that at low batch one request's KV is split over many workgroups whose
// partial results a second kernel merges.  Their stage counts are tuned for a 227/327 KiB
// shared-memory part with 212 SMs; the layout below is designed for gfx950 instead.
//
// Work decomposition.  A workgroup is four wavefronts, one per SIMD (a lone wave's 512
// registers hold a 32x512 fp32 output accumulator in AGPRs).  It owns 128 query rows
// (rows = (query token, head) pairs of one request; wave w takes rows 32w .. 32w+31) and one
// chunk of that request's tokens; every wave reads every KV tile of the chunk from LDS, so
// each KV byte crosses HBM and L2 once per 128 rows.
//
// KV staging.  A tile is 32 tokens x 576 bytes; a step is two tiles (64 tokens).  Tiles go
// HBM -> LDS with buffer_load ... lds (16 bytes per lane, no VGPR round trip) into an
// 8-tile ring (152 KiB of the CU's 160 KiB) = 4 step slots.  While the waves work on steps
// i - 1, i and i + 1 (see Schedule), step i + 2 is in flight.  Rows are stored with a
// 592-byte pitch (37 x 16 B); the 64-bank LDS then serves both read patterns below without
// conflicts.
// The buffer resource of each tile is bounded by the number of valid rows, so rows past
// the end of the sequence arrive as zeros: no NaN bytes from a page's unused tail can reach
// the P.V product (0 x NaN).  The query rows are staged through the same ring (in its last
// four tile slots, before the ring starts) and then held in registers.  Every DMA is issued
// from inline asm and waited on with explicit vmcnt counts: the compiler does not track
// them, so none of its own waits drain the ring (vector memory operations of its own, such
// as a register spill in the set-up, only make those counts wait longer, never shorter,
// since they complete in order).  M0 is written only by these asm statements (the compiler
// uses it for nothing else in this kernel).
//
// Math per step (per wave, 32 rows x 64 tokens), all on FP8 MFMA v_mfma_scale_f32_32x32x64:
//  * S^T = K . Q^T per tile: tokens along M, rows along N, 576 = 9 x 64 channels along K;
//    the two tiles' chains are interleaved.  Computing the transpose puts each lane's 16
//    scores for one row exactly where the P.V step needs them as an operand.  MFMA token m
//    reads LDS row perm_row(m), so register r of lane half gg holds tile token 2r + gg; the
//    permutation makes the transposed V reads below conflict-free.
//  * Online softmax in base 2 against a fixed reference max mu per row (the max of the row's
//    first step with a visible position), so the 256-register O is never rescaled.  Each
//    step's probabilities are normalised per row by 2^-e (e = floor of the row's step max
//    above mu) before the FP8 cast, and the MFMA's E8M0 scale multiplies them back by 2^e.
//    The two lanes that hold a row (n and n + 32) use the same e.  If a row's true max ends
//    up more than kHeadroom above mu (fp32 range at risk), the workgroup recomputes its
//    chunk once with mu = the true max.
//  * P is encoded as hi = e4m3(p) and lo = e4m3(p - hi), both in the same units, and
//    O^T += V^T . hi^T + V^T . lo^T as two MFMAs over the step's 64 tokens that share one V
//    operand (P.V with about 7 bits of P mantissa; a single e4m3 P costs several times the
//    2e-3 normalised-L1 budget against the fp64 oracle).  With V as the first operand the
//    accumulator holds O transposed: lane n owns row n, and each register four consecutive
//    value columns, so the epilogue stores 8 bytes per lane and instruction.
//  * V (the first 512 columns of the same tiles) is read transposed with ds_read_b64_tr_b8.
//
// Schedule.  A lone wave issues its instructions in order, and an MFMA keeps the matrix pipe
// busy for 64 clocks while the wave issues others behind it (measured: about eight VALU
// instructions, fewer transcendental, conversion or scalar ones).  Stage i of the pipeline
// runs the QK MFMAs of step i + 1, the softmax of step i and the P.V MFMAs of step i - 1,
// which are independent, interleaved as (PV hi, PV lo, QK) x 16, QK, QK: 50 MFMAs with all
// other work of the stage split into small pieces between them - fragment reads one or two
// MFMAs ahead of use, the address work and 10 DMA instructions of step i + 2 near the start,
// the softmax pieces over the rest.  One vmcnt wait and a barrier end the stage, after its
// last MFMA has issued.  Masking (sequence tail, causal positions, tiles past the chunk) is
// a uniform branch taken only in the last steps.
#include <type_traits>
#include <utility>

#include "internal.h"

namespace mla {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kPitch = 592;                 // LDS bytes per KV row (576 + one 16-B pad)
constexpr int kTileBytes = kTile * kPitch;  // 18944
constexpr int kSlot = kTileBytes + 512;     // guard for the half-used last DMA instruction
constexpr int kSlots = 8;                   // tile slots; a step takes two
constexpr int kStepSlots = kSlots / 2;
constexpr int kLds = kSlots * kSlot;        // 155648 bytes
constexpr int kLmin = 8;                    // fewest DMA instructions a wave issues per step
constexpr int kQSlot = 4;                   // the 128 query rows are staged in tile slots 4..7
constexpr int kQDma = 72;                   // 128 rows x 576 B / 1 KiB per DMA instruction
constexpr int kRows = 128;                  // query rows per workgroup
constexpr float kHeadroom = 64.0f;          // log2 range of a pass above its reference max
constexpr float kLog2PScale = 7.807354922057604f;  // log2(224): p in [0, 448)
constexpr float kLn2 = 0.6931471805599453f;

// MFMA token index -> LDS row of the tile: bits (b4 b3 b2 b1 b0) -> (b4 b3 b1 b0 b2).
__device__ __forceinline__ int perm_row(int m) {
  return (m & 0x18) | ((m & 3) << 1) | ((m >> 2) & 1);
}
// Index along M held in register r of a 32x32 MFMA result by lanes of half gg.
__device__ __forceinline__ int tok_of(int gg, int r) { return 8 * (r >> 2) + 4 * gg + (r & 3); }

// M0 = a + IMM: the LDS base of the DMA instructions that follow (with one wait state before
// the first of them).
template <int IMM>
__device__ __forceinline__ void set_m0(uint32_t a) {
  asm volatile("s_add_u32 m0, %0, %1\n\ts_nop 0" ::"s"(a), "n"(IMM) : "memory", "m0", "scc");
}
// One LDS DMA to M0 + OFF + 16 * lane from buffer offset voff + OFF (the instruction offset
// moves the LDS destination and the global source alike, and counts in the range check).
template <int OFF>
__device__ __forceinline__ void dma16_at(uint32_t voff, __amdgpu_buffer_rsrc_t rsrc) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:%2 lds" ::"v"(voff), "s"(rsrc), "n"(OFF)
               : "memory");
}
// 16 bytes per lane, global -> LDS at M0 + 16 * lane, with M0 = lds_addr + off (one wait
// state separates the M0 write from the DMA that reads it).
__device__ __forceinline__ void dma16_s(uint32_t lds_addr, uint32_t voff,
                                        __amdgpu_buffer_rsrc_t rsrc, uint32_t off) {
  asm volatile("s_add_u32 m0, %0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(off)
               : "memory", "m0", "scc");
}

// FP8 x FP8 32x32x64 MFMAs with explicit register classes: the scores live in VGPRs and O in
// AGPRs (left to itself the compiler puts every accumulator in AGPRs, which then do not
// hold O).  The "memory" clobber keeps the LDS fragment reads where the source places them.
// Hazards the compiler cannot see through the asm are handled here: the QK operands come
// straight from LDS reads (ordered by s_waitcnt, no VALU producer), a PV MFMA waits two
// states where its VALU-written scale may be fresh (see mfma_pv); a non-MFMA reader of an MFMA
// result is placed at least two MFMAs (128 clocks) after it or behind an explicit drain
// that takes the accumulators as operands (the compiler treats an asm output as ready at
// once and would otherwise copy it straight after the MFMA).
__device__ __forceinline__ f32x16 mfma_qk_first(const i32x8& a, const i32x8& b) {
  f32x16 d;
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %3 op_sel_hi:[0,0,0]"
               : "=&v"(d)
               : "v"(a), "v"(b), "v"(127)
               : "memory");
  return d;
}
__device__ __forceinline__ void mfma_qk(f32x16& d, const i32x8& a, const i32x8& b) {
  asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
               : "+v"(d)
               : "v"(a), "v"(b), "v"(127)
               : "memory");
}
// acc (O^T block) += V^T . P^T: A = V fragment (scale 2^0), B = P bytes (scale 2^(sb-127)).
// The first of a step waits two states for its freshly computed scale; the later ones read
// registers written long before.
template <bool kFirst>
__device__ __forceinline__ void mfma_pv(f32x16& acc, const i32x8& v, const i32x8& pbytes,
                                        int scale_b) {
  if constexpr (kFirst)
    asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                 : "+a"(acc)
                 : "v"(v), "v"(pbytes), "v"(127), "v"(scale_b)
                 : "memory");
  else
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                 : "+a"(acc)
                 : "v"(v), "v"(pbytes), "v"(127), "v"(scale_b)
                 : "memory");
}
__device__ __forceinline__ void mfma_drain2(f32x16& a, f32x16& b) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b)::"memory");
}
__device__ __forceinline__ void mfma_drain_acc(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc)::"memory");
}
// Orders later reads of acc after the preceding asm (no wait states of its own).
__device__ __forceinline__ void acc_fence(f32x16& acc) { asm volatile("" : "+a"(acc)); }

// max(a, b, c) in one v_max3_f32 (written out so no canonicalising v_max of each input is
// added; the inputs are MFMA results or -inf, never signalling NaNs).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// (value of lane n, value of lane n + 32) in every lane n and n + 32, by one
// v_permlane32_swap (no LDS traffic).
__device__ __forceinline__ f32x2 row_pair(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return (f32x2){__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// One accumulator block, copied to VGPRs where it is used.  The empty asm keeps the compiler
// from hoisting the copies of all 256 accumulator registers to one place, which would need
// more VGPRs than a wave has.
__device__ __forceinline__ f32x16 from_acc(const f32x16& a) {
  f32x16 v;
  asm volatile("" : "=v"(v) : "0"(a));
  return v;
}
// Keeps the compiler from moving instructions across this point (used to interleave VALU
// and LDS work with the MFMAs in source order).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ i32x4 lds_read16(const uint8_t* lds, uint32_t addr) {
  return *(const i32x4*)(lds + addr);
}

__device__ __forceinline__ i32x2 lds_read_tr8(uint8_t* lds, uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(lds + addr));
}

__device__ __forceinline__ i32x8 cat8(const i32x4& a, const i32x4& b) {
  return (i32x8){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// The four transposed 8-byte reads of a V fragment as one operand (built through a union:
// an element-wise build makes the compiler shuffle bytes).
union VFrag {
  i32x2 h[4];
  i32x8 v;
};

// Softmax state of one lane: its row's reference max, the running true max and its share of
// the row's sum of 2^(x - mu) * 224.
struct RowState {
  float mu, m_true, l_run;
};

// One step's scores (tile a, tile b), turned into probabilities in place.
struct Probs {
  f32x16 a, b;
  float off;   // exp2 argument offset
  float mpart; // running max over the scores (first max piece)
  float psum;  // running sum of the probabilities
  int ef;      // step exponent: P bytes are in units of 2^ef
};

// P bytes of a step: [tile a | tile b], hi and lo e4m3 terms.
struct PBytes {
  i32x8 hi, lo;
};

// What the P.V of a step needs: its P bytes and exponent.
struct StepP {
  PBytes pb;
  int ef;
};

// Calls f(std::integral_constant<int, i>{}) for i = 0 .. N-1 in order, so every index in
// the body is a compile-time constant (a #pragma unroll of a large body is not guaranteed).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Position of MFMA slot s of a pipeline stage among the MFMAs the stage issues: slots run
// (PV hi, PV lo, QK) x 16, QK, QK; a stage without QK or without PV skips those slots.  A
// stage opens with P.V, whose first V fragment was read before the previous stage's barrier,
// so the MFMA pipe restarts at once while the first K fragments are still on their way.
__host__ __device__ constexpr bool slot_is_qk(int s) { return s >= 48 || s % 3 == 2; }
__host__ __device__ constexpr int slot_gap(int s, bool qk, bool pv) {
  int g = -1;
  for (int t = 0; t <= s; ++t)
    if (slot_is_qk(t) ? qk : pv) ++g;
  return g;
}

// K fragments of one QK MFMA pair (tile a, tile b).
struct KPair {
  i32x4 a0, a1, b0, b1;
};

template <bool kPairPages, bool kDevScale, bool kRagged>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_kernel(const DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
  const uint32_t lds_base =
      (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)lds);

  // Every argument the set-up reads goes out in one batch of scalar loads and is waited for
  // once (left alone, the compiler issues them in three dependent rounds around the early
  // exit below, each a trip to the argument memory).
  asm volatile("" ::"s"(p.q8), "s"(p.page_table), "s"(p.seq_lens), "s"(p.batch),
               "s"(p.q_tokens), "s"(p.rows), "s"(p.page_size), "s"(p.max_pages),
               "s"(p.num_splits), "s"(p.groups), "s"(p.tiles_hint), "s"(p.div_splits.m),
               "s"(p.div_splits.s1), "s"(p.div_splits.s2), "s"(p.div_groups.m),
               "s"(p.div_groups.s1), "s"(p.div_groups.s2), "s"(p.div_tpp.m), "s"(p.div_tpp.s1),
               "s"(p.div_tpp.s2));
  asm volatile("" ::"s"(p.kv), "s"(p.page_bytes), "s"(p.div_heads.m), "s"(p.div_heads.s1),
               "s"(p.div_heads.s2), "s"(p.partial_o), "s"(p.partial_lse));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 31, gg = lane >> 5;

  // ---- workgroup -> (request, split, row group); the G row groups of one split share an
  // XCD (workgroups are dealt to the 8 XCDs round-robin) so their KV reads meet in one L2.
  const int G = p.groups, S = p.num_splits, M = p.rows;
  const int id = blockIdx.x;
  const int kx = id >> 3;
  const int kxg = (int)fast_div((uint32_t)kx, p.div_groups);
  const int g = kx - kxg * G;
  const int u = kxg * 8 + (id & 7);
  if (u >= p.batch * S) return;
  const int b_slot = (int)fast_div((uint32_t)u, p.div_splits), s = u - b_slot * S;
  // the request of this slot: slots are dispatched in order, so an order that puts the
  // longest requests first balances the CUs when lengths differ (values clamped into range)
  int b = b_slot;
  if constexpr (kRagged) {
    if (p.order) {
      b = ((const __attribute__((address_space(4))) int32_t*)p.order)[b_slot];
      b = b < 0 ? 0 : (b >= p.batch ? p.batch - 1 : b);
    }
  }

  // Wave-uniform scalars come from the constant address space (scalar loads, lgkmcnt).
  const __attribute__((address_space(4))) int32_t* seq_lens =
      (const __attribute__((address_space(4))) int32_t*)p.seq_lens;
  const __attribute__((address_space(4))) int32_t* page_table =
      (const __attribute__((address_space(4))) int32_t*)p.page_table;
  const int row0 = g * kRows;
  const uint32_t wave_lds = lds_base + (uint32_t)wave * 1024u;

  // ---- the workgroup's 128 query rows (contiguous in q8) go to tile slots 4..7 first: they
  // do not depend on the sequence length, so their DMA overlaps the length and page-table
  // loads below.  18 DMA instructions per wave; instruction i = wave + 4 j moves bytes
  // [1024 i, 1024 (i + 1)) of the rows.
  auto stage_q = [&]() __attribute__((always_inline)) {
    const int qrows = min(kRows, M - row0);
    const __amdgpu_buffer_rsrc_t qrsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.q8 + ((int64_t)b * M + row0) * kD), 0, qrows * kD, 0x00020000);
    const uint32_t qvoff = (uint32_t)wave * 1024u + 16u * (uint32_t)lane;
#pragma unroll
    for (int j = 0; j < kQDma / 4; ++j)
      dma16_s(wave_lds, qvoff + 4096u * j, qrsrc, kQSlot * kSlot + 4096 * j);
  };
  stage_q();
  // Prefetch the page-table entry of this chunk's first tile as it would be for a request of
  // the host's maximum length (exact for equal lengths), alongside the length itself.
  const __attribute__((address_space(4))) int32_t* ptrow = page_table + (int64_t)b * p.max_pages;
  const int pt_hint = ptrow[(uint32_t)min((int)fast_div((uint32_t)(s * p.tiles_hint), p.div_tpp),
                                          p.max_pages - 1)];
  int L = seq_lens[b];
  // query tokens of this request: all q_tokens, or its own count when requests differ; and
  // the request's context positions after the ones this call sees (a context shard other
  // than the last: the query tokens are the context's last positions, so every position
  // here is visible once that count reaches the query count)
  int qlen = p.q_tokens, after = 0;
  if constexpr (kRagged) {
    if (p.q_lens) qlen = ((const __attribute__((address_space(4))) int32_t*)p.q_lens)[b];
    if (p.ctx_after) after = ((const __attribute__((address_space(4))) int32_t*)p.ctx_after)[b];
    asm volatile("" ::"s"(L), "s"(pt_hint), "s"(qlen), "s"(after));  // all out together
    qlen = qlen < 0 ? 0 : (qlen > p.q_tokens ? p.q_tokens : qlen);
    after = after < 0 ? 0 : (after > p.q_tokens ? p.q_tokens : after);
  } else {
    asm volatile("" ::"s"(L), "s"(pt_hint));  // both loads go out before either is waited for
  }
  // scales kept on the device (written by an earlier kernel on the stream): loaded here, used
  // first by the softmax of step 0, long after they land
  float qs_dev = 0.f, ks_dev = 0.f;
  if constexpr (kDevScale) {
    qs_dev = *(const __attribute__((address_space(4))) float*)p.q_scale_dev;
    ks_dev = *(const __attribute__((address_space(4))) float*)p.kv_scale_dev;
  }
  const int Lmax = p.max_pages * p.page_size;
  L = L < 0 ? 0 : (L > Lmax ? Lmax : L);
  const int ntiles_all = (L + kTile - 1) / kTile;
  // tiles per split, rounded up to whole 64-token steps (so every chunk starts on an even tile)
  const int per = 2 * (int)fast_div((uint32_t)((ntiles_all + 1) / 2 + S - 1), p.div_splits);
  const int t_begin = s * per;
  const int ntiles = max(min(t_begin + per, ntiles_all) - t_begin, 0);

  const int64_t prow = (int64_t)(b * S + s) * M;  // first partial row of this (b, s)
  // nothing to compute: an empty chunk, or (per-request counts) a row group whose first row
  // already belongs to a query slot past the request's count, so every row of it is absent
  if (ntiles == 0 || (kRagged && (int)fast_div((uint32_t)row0, p.div_heads) >= qlen)) {
    wait_vmcnt<0>();  // the Q DMA lands before the workgroup's LDS is released
    for (int i = threadIdx.x; i < kRows; i += 256)
      if (row0 + i < M) p.partial_lse[prow + row0 + i] = -INFINITY;
    return;
  }

  const int P = p.page_size;
  const int tpp = P / kTile;  // tiles per page
  // page-table entry of the chunk's last tile
  const int pe_last = (int)fast_div((uint32_t)(t_begin + ntiles - 1), p.div_tpp);

  // ---- DMA lane offsets.  Of a tile's 19 one-KiB DMA chunks (LDS bytes 1024 c of the tile
  // slot), wave w moves chunks 4w .. 4w+3 with one M0 and instruction offsets 0, 1, 2, 3 KiB,
  // and waves 0..2 also chunk 16 + w.  The instruction offset moves the global source like the
  // LDS destination, so the lane offsets subtract it; tile resources start kPre bytes before
  // the tile (and reach kPre bytes further) so that every lane offset stays non-negative.
  // Lane l of chunk c is row (64c + l) / 37, 16-byte column (64c + l) % 37 of the LDS tile;
  // column 36 is the pad (it receives the next row's first 16 bytes, or zeros).
  constexpr uint32_t kPre = 128;
  uint32_t voff[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t c = i < 4 ? 4u * (uint32_t)wave + (uint32_t)i : 16u + (uint32_t)wave;
    const uint32_t pch = 64u * c + (uint32_t)lane;
    const uint32_t row = pch / 37u;
    voff[i] = 16u * (pch - row) + kPre - (i < 4 ? 1024u * (uint32_t)i : 0u);
  }
  const uint32_t m0_main = 4096u * (uint32_t)wave, m0_extra = 16384u + 1024u * (uint32_t)wave;

  // ---- page cursor: page-table entry and tile-within-page of tile 2j of the next step j
  // to prepare, advanced two tiles per step without divisions.  With an even number of tiles
  // per page (kPairPages) both tiles of a step lie in one page, since chunks start on even
  // tiles: one page-table load per step, and tile b's address is tile a's plus one tile.
  const int pe_first = (int)fast_div((uint32_t)t_begin, p.div_tpp);
  int cur_pe = pe_first;
  int cur_po = t_begin - cur_pe * tpp;
  struct StepPages {
    int page_a, po_a, page_b, po_b;
  };
  auto next_pages = [&]() __attribute__((always_inline)) -> StepPages {
    StepPages sp;
    sp.po_a = cur_po;
    sp.page_a = ptrow[(uint32_t)min(cur_pe, pe_last)];
    if constexpr (kPairPages) {
      sp.page_b = sp.page_a;
      sp.po_b = cur_po + 1;
      cur_po += 2;
      if (cur_po == tpp) {
        cur_po = 0;
        ++cur_pe;
      }
    } else {
      int pe_b = cur_pe, po_b = cur_po + 1;
      if (po_b >= tpp) { po_b = 0; ++pe_b; }
      sp.po_b = po_b;
      sp.page_b = ptrow[(uint32_t)min(pe_b, pe_last)];
      cur_po += 2;
      if (cur_po >= tpp) { cur_po -= tpp; ++cur_pe; }
      if (cur_po >= tpp) { cur_po -= tpp; ++cur_pe; }
    }
    return sp;
  };
  // rows of the chunk's tiles that lie before the chunk's end (and the sequence's) are loaded;
  // the rest of a slot, and every tile past the chunk, reads as zeros
  const int chunk_end = min(L, (t_begin + ntiles) * kTile);
  const int chunk_rows = chunk_end - t_begin * kTile;  // rows of the chunk from its first tile
  // bytes of tile ti (of the chunk) that are loaded: clamp(rows left, 0, 32) * 576, in SALU
  auto tile_bytes = [&](int ti) __attribute__((always_inline)) -> int {
    int r;
    asm("s_max_i32 %0, %1, 0\n\ts_min_i32 %0, %0, %2\n\ts_mul_i32 %0, %0, %3"
        : "=&s"(r)
        : "s"(chunk_rows - ti * kTile), "n"(kTile), "n"(kD)
        : "scc");
    return r;
  };
  auto make_rsrc = [&](const uint8_t* base, int nrec) __attribute__((always_inline)) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base - kPre), 0, nrec + (int)kPre,
                                             0x00020000);
  };
  auto tile_base = [&](int page, int po) __attribute__((always_inline)) -> const uint8_t* {
    if constexpr (kPairPages)  // page_bytes < 2^32: a 32 x 32 -> 64-bit product
      return p.kv + (uint64_t)(uint32_t)page * (uint32_t)p.page_bytes +
             (uint32_t)po * (uint32_t)(kTile * kD);
    else
      return p.kv + (uint64_t)(uint32_t)page * (uint64_t)p.page_bytes +
             (uint32_t)po * (uint32_t)(kTile * kD);
  };
  // buffer resources of the two tiles of step st
  // (in two halves, tile a then tile b, so that a pipeline stage can spread them over gaps)
  auto step_rsrc_a = [&](int st, const StepPages& sp, __amdgpu_buffer_rsrc_t& ra)
      __attribute__((always_inline)) -> const uint8_t* {
    const uint8_t* base_a = tile_base(sp.page_a, sp.po_a);
    ra = make_rsrc(base_a, tile_bytes(2 * st));
    return base_a;
  };
  auto step_rsrc_b = [&](int st, const StepPages& sp, const uint8_t* base_a,
                         __amdgpu_buffer_rsrc_t& rb) __attribute__((always_inline)) {
    if constexpr (kPairPages)
      rb = make_rsrc(base_a + kTile * kD, tile_bytes(2 * st + 1));
    else
      rb = make_rsrc(tile_base(sp.page_b, sp.po_b), tile_bytes(2 * st + 1));
  };
  auto step_rsrc = [&](int st, const StepPages& sp, __amdgpu_buffer_rsrc_t& ra,
                       __amdgpu_buffer_rsrc_t& rb) __attribute__((always_inline)) {
    step_rsrc_b(st, sp, step_rsrc_a(st, sp, ra), rb);
  };
  // DMA instructions i of tile slot j of a step slot (i = 4 only on waves 0..2)
  // (slot_lds: LDS address of the step slot; the two tiles of a step follow each other)
  auto tile_dma = [&](__amdgpu_buffer_rsrc_t rsrc, uint32_t slot_lds, auto jc, auto ic)
      __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value, i = decltype(ic)::value;
    if constexpr (i == 0) set_m0<j * kSlot>(slot_lds + m0_main);
    if constexpr (i < 4) dma16_at<1024 * i>(voff[i], rsrc);
    if constexpr (i == 4) {
      if (wave < 3) {
        set_m0<j * kSlot>(slot_lds + m0_extra);
        dma16_at<0>(voff[4], rsrc);
      }
    }
  };
  auto issue_tile = [&](__amdgpu_buffer_rsrc_t rsrc, uint32_t slot_lds, auto jc)
      __attribute__((always_inline)) {
    tile_dma(rsrc, slot_lds, jc, std::integral_constant<int, 0>{});
    tile_dma(rsrc, slot_lds, jc, std::integral_constant<int, 1>{});
    tile_dma(rsrc, slot_lds, jc, std::integral_constant<int, 2>{});
    tile_dma(rsrc, slot_lds, jc, std::integral_constant<int, 3>{});
    tile_dma(rsrc, slot_lds, jc, std::integral_constant<int, 4>{});
  };
  // Every step is issued, also past the end of the chunk (those load nothing and write zeros
  // into a free slot), so the number of DMA instructions in flight behind any step is fixed
  // and every wait below is a constant.
  auto slot_of = [&](int st) __attribute__((always_inline)) -> uint32_t {
    return lds_base + (uint32_t)((st % kStepSlots) * 2 * kSlot);
  };
  auto issue_step = [&](int st, const StepPages& sp) __attribute__((always_inline)) {
    __amdgpu_buffer_rsrc_t ra, rb;
    step_rsrc(st, sp, ra, rb);
    issue_tile(ra, slot_of(st), std::integral_constant<int, 0>{});
    issue_tile(rb, slot_of(st), std::integral_constant<int, 1>{});
  };

  // The first pass's steps 0 and 1 go out now, before the rest of the set-up: they are the
  // first KV the workgroup waits for, one HBM round trip away.
  const StepPages sp0 = next_pages();
  const StepPages sp1 = next_pages();
  issue_step(0, sp0);
  issue_step(1, sp1);

  const int wrow0 = row0 + wave * 32;
  const int R = wrow0 + n;  // this lane's query row (score, P and O layout)
  const bool row_ok = R < M;
  // last visible position of the row (bottom-right causal); rows past M are never stored
  // (computed for every lane, then selected: a branch here would make the compiler spill
  // around it and wait for the Q DMA)
  // A row whose query token t is past its request's count sees nothing (lim = -1), like a
  // query with no visible position: its lse is -inf.  Positions after the shard (ctx_after)
  // lift the causal limit past the shard's end, which is then the limit: rows of a tile past
  // L arrive as zeros and would otherwise count as scores of 0.
  const int t_r = (int)fast_div((uint32_t)R, p.div_heads);
  const int lim_r =
      kRagged ? (t_r < qlen ? min(L + after - qlen + t_r, L - 1) : -1) : L - qlen + t_r;
  const int lim = row_ok ? lim_r : 0x7FFFFFFF;
  int lim_min = min(L + after - qlen + (int)fast_div((uint32_t)wrow0, p.div_heads), L - 1);
  if constexpr (kRagged) {  // the wave's smallest limit is -1 if it holds an absent row
    const int t_hi = (int)fast_div((uint32_t)min(wrow0 + 31, M - 1), p.div_heads);
    if (t_hi >= qlen) lim_min = -1;
  }
  const int nsteps = (ntiles + 1) / 2;
  // Steps 0 .. nplain-1 need no masking: both tiles in the chunk and every position visible
  // to every row of this wave (tile 2j + 1 ends at (t_begin + 2j + 2) * 32 - 1 <= lim_min).
  int nplain;
  {
    const int jv = ((lim_min + 1) >> 5) - t_begin - 2;  // 2j <= jv
    nplain = __builtin_amdgcn_readfirstlane(min(jv < 0 ? 0 : jv / 2 + 1, ntiles / 2));
  }

  const int G16 = lane >> 4, i16 = lane & 15;
  const uint32_t vcol = 16 * (G16 & 1) + 8 * (i16 & 1);
  const uint32_t vrow0 = perm_row(tok_of(gg, i16 >> 1)) * kPitch + vcol;
  const uint32_t vrow1 = perm_row(tok_of(gg, 8 + (i16 >> 1))) * kPitch + vcol;
  const uint32_t krow = perm_row(n) * kPitch + 32 * gg;
  const float c2 = kDevScale ? score_scale_log2(qs_dev, ks_dev, p.softmax_scale) : p.c2;

  auto step_base = [&](int st) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)((st % kStepSlots) * 2 * kSlot);
  };

  i32x8 qf[9];  // Q fragments (B operand of S^T = K . Q^T), staged once per pass

  auto read_kpair = [&](uint32_t sb, int c) __attribute__((always_inline)) -> KPair {
    KPair k;
    k.a0 = lds_read16(lds, sb + krow + 64 * c);
    k.a1 = lds_read16(lds, sb + krow + 64 * c + 16);
    k.b0 = lds_read16(lds, sb + kSlot + krow + 64 * c);
    k.b1 = lds_read16(lds, sb + kSlot + krow + 64 * c + 16);
    return k;
  };

  RowState rs{-INFINITY, -INFINITY, 0.f};

  // ---- softmax pieces.  max_a / max_b find the row's step max (masking first when the step
  // needs it) and the step exponent, exp_piece(k) turns scores 2k, 2k+1 of [a | b] into
  // probabilities, hilo_pair encodes two probabilities as hi and lo e4m3 bytes.
  // Each piece ends in an empty asm that takes its results, so the compiler computes them
  // where the caller placed the piece (between two MFMAs) instead of next to their use.
  auto mask_tile = [&](f32x16& x, int ti) __attribute__((always_inline)) {
    // register r holds tile token 2 r + gg, visible while T0 + 2 r + gg <= lim, i.e. r <= c
    const int T0 = (t_begin + ti) * kTile;
    int c = ti < ntiles ? (lim - T0 - gg) >> 1 : -1;
    asm volatile("" : "+v"(c));  // keeps the compares inside the (rarely taken) masked branch
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = r > c ? -INFINITY : x[r];
  };
  // max of 16 scores as a tree of depth 3 (five, then two, then one v_max3_f32): a wave
  // issues in order, so a long dependent chain here would hold back the next MFMA
  auto max16 = [&](const f32x16& x, float extra) __attribute__((always_inline)) -> float {
    const float a0 = max3f(x[0], x[1], x[2]), a1 = max3f(x[3], x[4], x[5]);
    const float a2 = max3f(x[6], x[7], x[8]), a3 = max3f(x[9], x[10], x[11]);
    const float a4 = max3f(x[12], x[13], x[14]);
    const float b0 = max3f(a0, a1, a2), b1 = max3f(a3, a4, x[15]);
    return max3f(b0, b1, extra);
  };
  auto max_a = [&](Probs& t, int st, bool masked) __attribute__((always_inline)) {
    if (masked) mask_tile(t.a, 2 * st);
    t.mpart = max16(t.a, -INFINITY);
    asm volatile("" : "+v"(t.mpart));
  };
  auto max_b = [&](Probs& t, int st, bool masked) __attribute__((always_inline)) {
    if (masked) mask_tile(t.b, 2 * st + 1);
    t.mpart = max16(t.b, t.mpart);
    asm volatile("" : "+v"(t.mpart));
  };
  // the two halves of the row meet across lanes; the row's max in exp2 units
  auto max_row = [&](Probs& t) __attribute__((always_inline)) {
    const f32x2 both = row_pair(t.mpart);
    t.mpart = max3f(both[0], both[1], -INFINITY) * c2;  // c2 > 0
    asm volatile("" : "+v"(t.mpart));
  };
  auto step_exponent = [&](Probs& t) __attribute__((always_inline)) {
    const float mx = t.mpart;
    if (rs.mu == -INFINITY) rs.mu = mx;  // first step with a visible position
    rs.m_true = fmaxf(rs.m_true, mx);
    const float mref = rs.mu == -INFINITY ? 0.f : rs.mu;
    const float ef = fminf(fmaxf(floorf(mx - mref), -126.0f), 127.0f);
    t.ef = (int)ef;
    t.off = mref + ef - kLog2PScale;
    asm volatile("" : "+v"(t.off), "+v"(t.ef));
  };
  auto exp_piece = [&](Probs& t, int k) __attribute__((always_inline)) {
    // p = 2^(c2 s - off), in [0, 448); 0 where masked
    float x0, x1;
    if (k < 8) {
      x0 = t.a[2 * k] = __builtin_amdgcn_exp2f(fmaf(t.a[2 * k], c2, -t.off));
      x1 = t.a[2 * k + 1] = __builtin_amdgcn_exp2f(fmaf(t.a[2 * k + 1], c2, -t.off));
    } else {
      x0 = t.b[2 * k - 16] = __builtin_amdgcn_exp2f(fmaf(t.b[2 * k - 16], c2, -t.off));
      x1 = t.b[2 * k - 15] = __builtin_amdgcn_exp2f(fmaf(t.b[2 * k - 15], c2, -t.off));
    }
    t.psum = (k == 0 ? x0 : t.psum + x0) + x1;
    asm volatile("" : "+v"(t.psum));
    if (k == 15) rs.l_run += ldexpf(t.psum, t.ef);
  };
  // hi/lo bytes of probabilities o, o + 1 of tile v, which fill half (high or low) of word q of
  // the step's P bytes.  The low half comes first and starts the word in a free register (an
  // empty asm names it; its old contents are overwritten by the high half next).
  auto hilo_pair = [&](const f32x16& v, int o, int q, auto hc, PBytes& pb)
      __attribute__((always_inline)) {
    constexpr bool high = decltype(hc)::value;
    int w = pb.hi[q], w2 = pb.lo[q];
    if (!high) {
      asm volatile("" : "=v"(w));
      asm volatile("" : "=v"(w2));
    }
    w = __builtin_amdgcn_cvt_pk_fp8_f32(v[o], v[o + 1], w, high);
    const f32x2 dh = __builtin_amdgcn_cvt_pk_f32_fp8(w, high);
    w2 = __builtin_amdgcn_cvt_pk_fp8_f32(v[o] - dh[0], v[o + 1] - dh[1], w2, high);
    asm volatile("" : "+v"(w), "+v"(w2));  // computed here, not sunk next to the PV MFMAs
    pb.hi[q] = w;
    pb.lo[q] = w2;
  };
  f32x16 o[16];  // O^T blocks: register r of block d = row wrow0 + n, column 32 d + tok_of(gg, r)

  // K fragment of QK MFMA q of a step (tile q & 1, channel block q >> 1).
  auto read_k = [&](uint32_t sb, int q) __attribute__((always_inline)) -> i32x8 {
    const uint32_t a = sb + (uint32_t)((q & 1) * kSlot) + krow + 64u * (uint32_t)(q >> 1);
    return cat8(lds_read16(lds, a), lds_read16(lds, a + 16));
  };
  // V fragment of value block d of a step: four transposed 8-byte reads.
  auto read_v = [&](uint32_t sb, int d, i32x2 (&va)[4]) __attribute__((always_inline)) {
    va[0] = lds_read_tr8(lds, sb + vrow0 + 32 * d);
    va[1] = lds_read_tr8(lds, sb + vrow1 + 32 * d);
    va[2] = lds_read_tr8(lds, sb + kSlot + vrow0 + 32 * d);
    va[3] = lds_read_tr8(lds, sb + kSlot + vrow1 + 32 * d);
  };
  // Softmax of a step in kPieces pieces: 0 max over tile a, 1 max over tile b, 2 the row's
  // max across the lane halves, 3 step exponent, 4..19 exp2 of scores 2j, 2j+1 of [a | b],
  // 20..35 their hi/lo bytes.
  constexpr int kPieces = 36;
  auto softmax_piece = [&](Probs& t, int st, bool masked, int k, StepP& out)
      __attribute__((always_inline)) {
    if (k == 0) max_a(t, st, masked);
    else if (k == 1) max_b(t, st, masked);
    else if (k == 2) max_row(t);
    else if (k == 3) step_exponent(t);
    else if (k <= 19) exp_piece(t, k - 4);
    else if (k - 20 < 8 && (k & 1) == 0)
      hilo_pair(t.a, 2 * (k - 20), (k - 20) >> 1, std::false_type{}, out.pb);
    else if (k - 20 < 8)
      hilo_pair(t.a, 2 * (k - 20), (k - 20) >> 1, std::true_type{}, out.pb);
    else if ((k & 1) == 0)
      hilo_pair(t.b, 2 * (k - 28), (k - 20) >> 1, std::false_type{}, out.pb);
    else
      hilo_pair(t.b, 2 * (k - 28), (k - 20) >> 1, std::true_type{}, out.pb);
    if (k == kPieces - 1) out.ef = t.ef;
  };

  // One pipeline stage st: the QK MFMAs of step st + 1 (scores into sn, when kQK), the softmax
  // of step st (scores sc -> P bytes pn) and the P.V MFMAs of step st - 1 (P bytes pp, when
  // kPV).  The three are independent, so the MFMAs interleave as (PV hi, PV lo, QK) x 16, QK,
  // QK and every gap between two MFMAs carries an even share of the softmax pieces, the K and
  // V fragment reads and the DMA of step st + 2.  Ends with the first V fragment of step st
  // read for the next stage, every DMA landed and a barrier.
  StepPages sp_next;  // pages of the next step to issue
  i32x2 vnext[4];     // V fragment of block 0 of the step the next stage multiplies
  // mask_c: whether step st may need masking (false only where the caller knows st < nplain,
  // so the plain steps carry no masking branch at all).
  auto stage = [&](int st, Probs& sc, Probs& sn, const StepP& pp, StepP& pn, auto qk_c,
                   auto pv_c, auto mask_c) __attribute__((always_inline)) {
    constexpr bool kQK = decltype(qk_c)::value, kPV = decltype(pv_c)::value;
    static_assert(kQK || kPV, "a stage issues MFMAs");
    constexpr int nmf = (kQK ? 18 : 0) + (kPV ? 32 : 0);
    const bool masked = decltype(mask_c)::value && st >= nplain;
    const uint32_t sbk = step_base(st + 1), sbv = step_base(st + 3);  // (st - 1) mod 4
    const int escale = 127 + pp.ef;
    const uint32_t slot2 = slot_of(st + 2);
    i32x8 kf[18];
    i32x2 va[16][4];
    __amdgpu_buffer_rsrc_t ra, rb;
    const uint8_t* base_next;
    // K fragment of the first QK (the second follows behind the first MFMA, unless the stage
    // opens with QK)
    if constexpr (kQK) kf[0] = read_k(sbk, 0);
    if constexpr (kQK && !kPV) kf[1] = read_k(sbk, 1);
    if constexpr (kPV) {
      va[0][0] = vnext[0];
      va[0][1] = vnext[1];
      va[0][2] = vnext[2];
      va[0][3] = vnext[3];
    }
    // work between MFMA number G and the next one
    auto gap = [&](auto gc) __attribute__((always_inline)) {
      constexpr int G = decltype(gc)::value;
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;
      using I4 = std::integral_constant<int, 4>;
      sched_fence();
      // the ten DMA instructions (five per tile), one per gap from the stage's first MFMA on:
      // the slot they fill was released by the previous stage's barrier, and the sooner they
      // are issued the more of the stage hides their HBM latency before the wait at its end
      constexpr auto dma_gap = [](int i) { return i + 1; };
      // behind the stage's first MFMA: the second K fragment and the resource of tile a of
      // step st + 2 (whose DMA goes into the slot step st - 2 left); tile b's three gaps on
      if constexpr (G == 0) {
        if constexpr (kQK && kPV) kf[1] = read_k(sbk, 1);
        base_next = step_rsrc_a(st + 2, sp_next, ra);
      }
      if constexpr (G == 3) step_rsrc_b(st + 2, sp_next, base_next, rb);
      if constexpr (G == dma_gap(0)) tile_dma(ra, slot2, I0{}, I0{});
      if constexpr (G == dma_gap(1)) tile_dma(ra, slot2, I0{}, I1{});
      if constexpr (G == dma_gap(2)) tile_dma(ra, slot2, I0{}, I2{});
      if constexpr (G == dma_gap(3)) tile_dma(ra, slot2, I0{}, I3{});
      if constexpr (G == dma_gap(4)) tile_dma(ra, slot2, I0{}, I4{});
      if constexpr (G == dma_gap(5)) tile_dma(rb, slot2, I1{}, I0{});
      if constexpr (G == dma_gap(6)) tile_dma(rb, slot2, I1{}, I1{});
      if constexpr (G == dma_gap(7)) tile_dma(rb, slot2, I1{}, I2{});
      if constexpr (G == dma_gap(8)) tile_dma(rb, slot2, I1{}, I3{});
      if constexpr (G == dma_gap(9)) tile_dma(rb, slot2, I1{}, I4{});
      static_assert(10 < nmf, "every DMA instruction has a gap");
      // softmax pieces k with 1 + floor(k (nmf - 1) / kPieces) == G (gap 0 holds the address work)
      static_for<kPieces>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        if constexpr (1 + (k * (nmf - 1)) / kPieces == G) softmax_piece(sc, st, masked, k, pn);
      });
      sched_fence();
    };
    static_for<50>([&](auto sc_) __attribute__((always_inline)) {
      constexpr int slot = decltype(sc_)::value;
      constexpr int G = slot_gap(slot, kQK, kPV);
      if constexpr (slot_is_qk(slot)) {
        if constexpr (kQK) {
          constexpr int q = slot >= 48 ? slot - 32 : slot / 3;  // 0..17
          if constexpr (q == 0) sn.a = mfma_qk_first(kf[q], qf[0]);
          else if constexpr (q == 1) sn.b = mfma_qk_first(kf[q], qf[0]);
          else if constexpr ((q & 1) != 0) mfma_qk(sn.b, kf[q], qf[q >> 1]);
          else mfma_qk(sn.a, kf[q], qf[q >> 1]);
          // every fragment read follows the MFMA before it, so the MFMA issues first
          if constexpr (q + 2 < 18) kf[q + 2] = read_k(sbk, q + 2);
          gap(std::integral_constant<int, G>{});
        }
      } else {
        if constexpr (kPV) {
          constexpr int d = slot / 3;
          constexpr bool hi = slot % 3 == 0;
          VFrag vf;
          vf.h[0] = va[d][0];
          vf.h[1] = va[d][1];
          vf.h[2] = va[d][2];
          vf.h[3] = va[d][3];
          if constexpr (hi && d == 0) mfma_pv<true>(o[d], vf.v, pp.pb.hi, escale);
          else if constexpr (hi) mfma_pv<false>(o[d], vf.v, pp.pb.hi, escale);
          else mfma_pv<false>(o[d], vf.v, pp.pb.lo, escale);
          if constexpr (hi && d + 1 < 16) read_v(sbv, d + 1, va[d + 1]);
          gap(std::integral_constant<int, G>{});
        }
      }
    });
    // V block 0 of step st for the next stage (its slot is not a DMA target until then); pages
    // of step st + 3 (scalar loads, waited for after the barrier); every DMA so far has landed
    // and every wave is past this stage's reads
    read_v(step_base(st), 0, vnext);
    sp_next = next_pages();
    wait_vmcnt<0>();
    // A bare s_barrier: this wave's DMA writes have landed (vmcnt above) and every LDS read of
    // the slot the next DMA overwrites was consumed by this stage's MFMAs, so no LDS or scalar
    // load needs to drain first (a __syncthreads() fence would wait for them all here).
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::"s"(sp_next.page_a), "s"(sp_next.page_b));
  };
  // P.V of the last step, with nothing else to overlap.
  auto last_pv = [&](int st, const StepP& pp) __attribute__((always_inline)) {
    const uint32_t sbv = step_base(st);
    const int escale = 127 + pp.ef;
    i32x2 va[16][4];
    read_v(sbv, 0, va[0]);
    static_for<16>([&](auto dc) __attribute__((always_inline)) {
      constexpr int d = decltype(dc)::value;
      if constexpr (d + 1 < 16) read_v(sbv, d + 1, va[d + 1]);
      VFrag vf;
      vf.h[0] = va[d][0];
      vf.h[1] = va[d][1];
      vf.h[2] = va[d][2];
      vf.h[3] = va[d][3];
      if constexpr (d == 0) mfma_pv<true>(o[d], vf.v, pp.pb.hi, escale);
      else mfma_pv<false>(o[d], vf.v, pp.pb.hi, escale);
      mfma_pv<false>(o[d], vf.v, pp.pb.lo, escale);
    });
  };

#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    rs.l_run = 0.f;
    // ---- the query rows and steps 0 and 1 (issued above for the first pass; again for a
    // second pass, since the Q fragments are live within a pass only), the same order
    if (pass > 0) {
      cur_pe = pe_first;
      cur_po = t_begin - cur_pe * tpp;
      stage_q();
      const StepPages spa = next_pages();
      const StepPages spb = next_pages();
      issue_step(0, spa);
      issue_step(1, spb);
    }
    sp_next = next_pages();  // step 2, issued by stage 0
#pragma unroll
    for (int d = 0; d < 16; ++d) o[d] = (f32x16){0.f};  // while the DMAs are in flight
    wait_vmcnt<2 * kLmin>();  // this wave's Q chunks have landed
    __syncthreads();
    {
      const uint32_t qrow = (uint32_t)(kQSlot * kSlot + (wave * 32 + n) * kD + 32 * gg);
#pragma unroll
      for (int c = 0; c < 9; ++c)
        qf[c] = cat8(lds_read16(lds, qrow + 64 * c), lds_read16(lds, qrow + 64 * c + 16));
    }
    wait_vmcnt<kLmin>();  // step 0 has landed (step 1 may still be in flight)
    __syncthreads();      // ... for every wave; the Q slots are free from here on

    // ---- step 0's scores, not overlapped with anything
    Probs X, Y;
    StepP PA, PB;
    {
      const uint32_t sb = step_base(0);
#pragma unroll
      for (int c = 0; c < 9; ++c) {
        const KPair k = read_kpair(sb, c);
        if (c == 0) {
          X.a = mfma_qk_first(cat8(k.a0, k.a1), qf[0]);
          X.b = mfma_qk_first(cat8(k.b0, k.b1), qf[0]);
        } else {
          mfma_qk(X.a, cat8(k.a0, k.a1), qf[c]);
          mfma_qk(X.b, cat8(k.b0, k.b1), qf[c]);
        }
      }
      mfma_drain2(X.a, X.b);
    }
    wait_vmcnt<0>();  // step 1 has landed
    __syncthreads();

    // ---- the pipeline.  Invariant at the top of the loop: scores of step st in Y, P bytes
    // of step st - 1 in PA.
    // (a single-step chunk computes the scores of an empty step 1 here, unused)
    using T = std::true_type;
    using F = std::false_type;
    stage(0, X, Y, PB, PA, T{}, F{}, T{});
    int st = 1;
    for (; st + 2 <= nsteps - 1; st += 2) {
      stage(st, Y, X, PA, PB, T{}, T{}, T{});
      stage(st + 1, X, Y, PB, PA, T{}, T{}, T{});
    }
    if (st <= nsteps - 2) {
      stage(st, Y, X, PA, PB, T{}, T{}, T{});
      ++st;
      Y = X;
      PA = PB;
    }
    if (nsteps >= 2) {  // softmax of the last step beside the P.V of the one before
      stage(nsteps - 1, Y, X, PA, PB, F{}, T{}, T{});
      PA = PB;
    }
    last_pv(nsteps - 1, PA);
    mfma_drain_acc(o[15]);
#pragma unroll
    for (int d = 0; d < 15; ++d) acc_fence(o[d]);
    wait_vmcnt<0>();  // the steps past the chunk have landed too
    // all waves are past their last read of the ring; decide whether to recompute
    const bool over = rs.mu != -INFINITY && rs.m_true > rs.mu + kHeadroom;
    if (!__syncthreads_or(over)) break;
    // second pass: reference = the row's true max, so every exponent is <= 0
    rs.mu = rs.m_true;
  }

  // ---- normalise, write partial O (fp16, in units of kv_scale: |O| <= 448) and lse
  const float mu = rs.mu;
  const f32x2 lpair = row_pair(rs.l_run);
  const float Ls = lpair[0] + lpair[1];  // both halves of the row
  const float f = (mu != -INFINITY && Ls > 0.f) ? 1.0f / Ls : 0.f;
  if (lane < 32 && row_ok)
    p.partial_lse[prow + R] = Ls > 0.f ? (mu + log2f(Ls) - kLog2PScale) * kLn2 : -INFINITY;
  // Transpose through LDS (free now: every DMA has landed and every wave is past the ring) so
  // that each store instruction writes one whole 1 KiB partial row: this wave's 32 rows x 512
  // columns go to LDS rows of kOPitch bytes (registers 4k .. 4k+3 of block d hold columns
  // 32 d + 8 k + 4 gg + 0..3 of row n), then lane l stores columns 8 l .. 8 l + 7 of a row.
  constexpr int kOPitch = 1040;  // 16-byte aligned; 2-way bank conflicts on the 8-byte writes
  uint8_t* ob = lds + wave * (32 * kOPitch);
#pragma unroll
  for (int d = 0; d < 16; ++d) {
    const f32x16 v = from_acc(o[d]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      typedef _Float16 h4 __attribute__((ext_vector_type(4)));
      const h4 h = {(_Float16)(v[4 * k] * f), (_Float16)(v[4 * k + 1] * f),
                    (_Float16)(v[4 * k + 2] * f), (_Float16)(v[4 * k + 3] * f)};
      *(uint2*)(ob + n * kOPitch + 2 * (32 * d + 8 * k + 4 * gg)) = __builtin_bit_cast(uint2, h);
    }
  }
  _Float16* orow = (_Float16*)p.partial_o + (prow + wrow0) * kDv + 8 * lane;
  const int nrows = min(32, M - wrow0);
#pragma unroll
  for (int r = 0; r < 32; ++r)
    if (r < nrows) *(uint4*)(orow + r * kDv) = *(const uint4*)(ob + r * kOPitch + 16 * lane);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int rows_per_group, hipStream_t s) {
  clear_last_error();
  if (rows_per_group != kRows) return hipErrorInvalidValue;
  const int64_t units = (int64_t)p.batch * p.num_splits;
  const int64_t blocks = ((units + 7) / 8) * 8 * p.groups;
  // an even number of tiles per page (and pages under 4 GiB) takes the paired-tile cursor
  const bool paired = (p.page_size / kTile) % 2 == 0 && p.page_bytes < (int64_t(1) << 32);
  const int v = (paired ? 1 : 0) | (p.q_scale_dev != nullptr ? 2 : 0) |
                (p.q_lens || p.ctx_after || p.order ? 4 : 0);
  const dim3 grid((unsigned)blocks), block(256);
  switch (v) {
    case 0: decode_kernel<false, false, false><<<grid, block, 0, s>>>(p); break;
    case 1: decode_kernel<true, false, false><<<grid, block, 0, s>>>(p); break;
    case 2: decode_kernel<false, true, false><<<grid, block, 0, s>>>(p); break;
    case 3: decode_kernel<true, true, false><<<grid, block, 0, s>>>(p); break;
    case 4: decode_kernel<false, false, true><<<grid, block, 0, s>>>(p); break;
    case 5: decode_kernel<true, false, true><<<grid, block, 0, s>>>(p); break;
    case 6: decode_kernel<false, true, true><<<grid, block, 0, s>>>(p); break;
    default: decode_kernel<true, true, true><<<grid, block, 0, s>>>(p); break;
  }
  return hipGetLastError();
}

}  // namespace mla
