// Paged causal prefill for gfx950 on bf16 MFMA (fp32 accumulation).
//
// What is computed ("[None][feat] Run Gemma4 head_dim 512 attention on Triton",
// TensorRT-LLM pull request 17772, section "Approach": causal attention when no custom mask
// is given over FlashInfer's HND paged layout; section "Not covered": the current tokens
// versus the cached prefix): the q_len new tokens of a request are its last keys, row i
// sits at position L - q_len + i and attends keys t <= position (and t > position - W with
// a sliding window).  head_dim_qk = 512 with head_dim_vo = 256 reads V from its own pool
// ("feat(attention): asymmetric VO-split NVFP4 paged prefill (qk=512/vo=256) for Gemma-4
// on SM120/121", FlashInfer pull request 3684, section "Summary").
//
// Work decomposition.  A tile is 128 query rows of one (request, KV head): the (token,
// head) pairs of the head group, flattened token-major, so the G heads that share a KV
// head share every K/V tile.  One workgroup of 8 waves runs a tile; each wave owns 16 rows.
// Keys stream through LDS in stages of 32 (K double-buffered, V triple-buffered, filled by
// direct-to-LDS copies from the pages).  Per stage and wave, with v_mfma_f32_16x16x32_bf16:
//   * S^T = K Q^T (keys on M, the wave's 16 rows on N, head_dim on K): A = K rows from LDS,
//     B = Q held in registers for the whole tile.  In the output layout every lane holds
//     8 scores of one query row, so the online softmax of a row lives in one lane group.
//   * O^T += V^T P^T (head_dim on M, rows on N, keys on K): B = P straight from the score
//     registers (same lane, same key order), A = V read transposed from LDS.  The O^T
//     accumulators of a lane again all belong to its own row.
//   * The two waves sharing a SIMD run the stage's phases in rotated order, so one's
//     softmax overlaps the other's MFMAs.
//   * The running max is only moved when a row's max grows by more than 2^8, so the
//     accumulators are rescaled rarely; the final normalisation uses the same reference
//     max, so the result is unchanged.
// Every wave reads the whole K and V stage from LDS (64 KB at 512/512) for its 16 rows: 1 KB
// of LDS reads per 16-clock MFMA, so the MFMA pipes run only as fast as the LDS delivers
// (measured per CU: ~230 B per clock for 16-byte reads, ~150 for the 8-byte and
// transposing reads that V takes) and as its latency is hidden.
// FP8 E4M3FN KV (the Triton page, section "Approach": FP8 caches are cast on load by the
// same kernels in both phases): the stages hold the codes themselves, copied direct to LDS
// like bf16 rows (half the bytes).  V operands are widened to bf16 in registers (exact)
// after each LDS read (ds_read_b64_tr_b8, 8 keys of one dim); S^T runs on the FP8 MFMA
// with the K codes as they are and Q as two E4M3 terms (see qk).  NVFP4 KV (the FlashInfer page, sections "Summary"
// and "What's in it": packed E2M1 with one E4M3 block scale per 16 head_dim elements): a
// direct-to-LDS copy cannot convert, so each wave loads its key rows' codes and block
// scales into registers and writes them to LDS as bf16 (exact), in the same swizzled
// layout, before the barrier that hands the stage over.  k_scale folds into the score
// scale and v_scale into the final normalisation.
// The score scale may have any sign: the kernel works with |scale| and flips the sign bits
// of Q when the scale is negative (a zero scale zeroes Q, so every visible key weighs the
// same), so masks and running maxima are taken on scores that grow with the scaled ones.

#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>
#include <utility>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

constexpr int kKeyStage = kPrefillKeyStage;  // keys per LDS stage
constexpr float kRescaleThreshold = 8.0f;  // log2 units

// How a stage's key rows are found in the pages.
constexpr int kPagesAny = 0;    // any page size: one page-table lookup per key row
constexpr int kPagesPow2 = 1;   // power-of-two page size below 32: same, with shifts
constexpr int kPagesStage = 2;  // page size a multiple of 32: a stage lies in one page

struct PrefillArgs {
  const uint16_t* q;          // [total_q, Hq, DQK] bf16
  const char* k;
  const char* v;
  int64_t k_sp, k_sh, k_st;   // byte strides (page, head, token)
  int64_t v_sp, v_sh, v_st;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const PrefillItem* items;
  void* out;                  // [total_q, Hq, out_stride], this launch's DVO columns first
  int32_t out_stride;         // elements between output rows (DVO, or the whole head_dim
                              // when a launch computes one part of it)
  float* lse;                 // [total_q, Hq] or null
  float* part_o;              // split tiles: [slot][kv head][tile row][DVO] fp32
  float* part_lse;            // [slot][kv head][tile row][2] fp32, log2 domain
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t page_size;
  int32_t page_shift;         // log2(page_size) when it is a power of two
  int32_t window;             // 0 = none
  int32_t causal;
  int32_t out_fp32;
  float scale_log2;           // |sm_scale * k_scale| * log2(e) (1 * log2(e) for a zero scale)
  uint32_t q_and;             // applied to every Q dword: zero for a zero scale
  uint32_t q_xor;             // then this: the bf16 sign bits for a negative scale
  float v_scale;              // FP8 / NVFP4: tensor-wide V scale (1 for bf16)
  const char* k_sf;           // NVFP4 block scales, else null
  const char* v_sf;
  int64_t ks_sp, ks_sh, ks_st;  // block-scale byte strides
  int64_t vs_sp, vs_sh, vs_st;
};

// LDS stages hold key rows unpadded; 16-byte chunk c of row r sits at chunk position
// c ^ swz(r).  The K swizzle spreads the 16 rows a K-operand read touches over all banks;
// the V swizzle (even values, so 32-byte pairs stay together) spreads the 4 key rows of a
// transpose read and its neighbouring lane block.
__device__ __forceinline__ int k_swz(int row) { return row & 15; }
__device__ __forceinline__ int v_swz(int row) { return 2 * (row & 7); }
// FP8 stages: a V-operand read (ds_read_b64_tr_b8) touches key rows 4g .. 4g+3 and
// 16+4g .. 16+4g+3 of a lane block g at one chunk; this swizzle gives each of the 16 rows
// of two neighbouring blocks its own chunk position.
__device__ __forceinline__ int v_swz_fp8(int row) { return (row & 7) | ((row & 16) >> 1); }

// Waits until at most N of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Calls f(integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time.
template <int... I, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

// ds_read_b64_tr_b16 at LDS byte address addr + OFF, as inline assembly: the compiler does
// not count it, so the caller waits for it with lds_wait<N>.  (Issued through the builtin,
// the compiler cannot tell which LDS buffer the read touches and makes it wait for every
// direct-to-LDS copy in flight, including the next stage's.)
template <int OFF>
__device__ __forceinline__ u32x2_t lds_read_tr16_at(uint32_t addr) {
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
// ds_read_b64_tr_b8, likewise: within each 16-lane block, lane 8c + e receives byte e of
// the 8-byte segments addressed by lanes c, c + 2, .., c + 14 (in that order; measured on
// the GPU with an in-bounds probe).
template <int OFF>
__device__ __forceinline__ u32x2_t lds_read_tr8_at(uint32_t addr) {
  u32x2_t r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
  return r;
}
// Waits until at most N LDS (or scalar memory) operations of this wave are outstanding.
// The registers that the awaited reads fill pass through the statement, so the compiler
// cannot use or copy them before it.
template <int N>
__device__ __forceinline__ void lds_wait(u32x2_t& a, u32x2_t& b) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(u32x2_t& a) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a) : "n"(N));
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Eight FP8 E4M3FN codes (byte i = element i) as eight bf16 values, exact (every E4M3FN
// value is a bf16 value); the conversion's scale operand is 1.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(u32x2_t c) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[0], 1.0f, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[0], 1.0f, true);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[1], 1.0f, false);
  const auto e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)c[1], 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
}

// Page and slot of a wave-uniform logical token, through a scalar load.
template <bool POW2>
__device__ __forceinline__ void uniform_page_slot(const int32_t* pages, int t, int page_size,
                                                  int page_shift, int& page, int& slot) {
  const_i32_ptr cp = (const_i32_ptr)pages;
  t = __builtin_amdgcn_readfirstlane(t);
  int j;
  if constexpr (POW2) {
    j = t >> page_shift;
    slot = t & (page_size - 1);
  } else {
    j = t / page_size;
    slot = t - j * page_size;
  }
  page = cp[j];
}

// Raw buffer resource at base p: no stride, no bound (every offset the kernel forms stays
// inside the page it addresses), 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* p) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, -1, 0x00020000);
}

__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// SHORT: the form for plans rich in short tiles, whose waves without rows skip the
// arithmetic (below); kept apart because the branch costs full tiles ~2 % (register
// assignment and scheduling of the whole kernel shift with it).
template <int DQK, int DVO, int PM, int KV, bool SHORT>
__global__ __launch_bounds__(512, 2) void prefill_kernel(PrefillArgs a) {
  constexpr bool FP4 = KV == kKvFp4;
  constexpr bool CONV = FP4;                // stages pass through registers and are converted
  constexpr bool F8 = KV == kKvFp8;         // stages hold the FP8 codes; operands widen after the read
  // FP8 S^T on the FP8 MFMA (K codes as they are, Q in two E4M3 terms), except at 512/512
  // with per-row page lookups, whose addressing leaves no registers for it (it spilled);
  // there K widens to bf16 like V.
  constexpr bool F8MF = F8 && (PM == kPagesStage || DQK != 512 || DVO != 512);
  constexpr int EB = F8 ? 1 : 2;            // bytes per staged element
  constexpr int NW = kPrefillWaves;
  constexpr int KS = kKeyStage;
  constexpr int QSTEPS = DQK / 32;          // MFMA K-steps of S^T
  constexpr int OT = DVO / 16;              // 16-wide head_dim tiles of O^T
  constexpr int KCH = DQK * EB / 16;        // 16-byte chunks per K row
  constexpr int VCH = DVO * EB / 16;
  constexpr int KRPI = 64 / KCH;            // K rows per copy instruction (1, 2 or 4)
  constexpr int VRPI = 64 / VCH;
  constexpr int RPW = KS / NW;              // key rows each wave copies per stage
  static_assert(RPW == 4, "each wave copies four key rows per stage");
  // Read-ahead of the software pipelines (steps of S^T, tiles of O^T), bounded by the
  // registers left beside Q (DQK / 8 per lane) and O (DVO / 4 per lane).  Two steps of K at
  // 512/512 fit in 253 VGPRs and measured ~1 % faster than one; the NVFP4 kernel, which
  // also holds a stage's codes in registers, keeps one.  FP8 V tiles are half as wide in
  // registers (read-ahead depths 2 to 6 of either measured within 1 %).
  constexpr int KD = DVO == 512 ? (CONV ? 1 : 2) : 4;
  constexpr int VD = DVO == 512 ? (F8 ? 4 : 2) : 4;

  // K stages are double-buffered, V stages triple-buffered: half of the waves use a stage's
  // V one interval after its K (see the stage loop below).  One array per K buffer: the
  // compiler then sees that K reads of one buffer do not alias the direct-to-LDS copies into
  // the other, and does not make them wait for those copies (V is read by inline assembly,
  // which the compiler does not track).  1 KB alignment: the swizzled read addresses below
  // differ from a per-lane base only in bits the base leaves zero, so one XOR forms each.
  using st_t = typename std::conditional<F8, uint8_t, uint16_t>::type;  // staged element
  constexpr int VSTAGE = KS * DVO;  // elements of one V buffer
  __shared__ __attribute__((aligned(1024))) st_t k_lds0[KS * DQK], k_lds1[KS * DQK];
  __shared__ __attribute__((aligned(1024))) st_t v_lds[3 * VSTAGE];
  auto k_buf = [&](auto slot_c) -> st_t* { if constexpr (decltype(slot_c)::value == 0) return k_lds0; else return k_lds1; };
  auto vswz = [](int row) { return F8 ? v_swz_fp8(row) : v_swz(row); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;   // k-slot group of the MFMA operands
  const int n = lane & 15;    // this lane's query row within the wave (and operand row)
  const int hkv = a.num_kv_heads;
  const int kvh = blockIdx.x % hkv;
  const PrefillItem it = a.items[blockIdx.x / hkv];
  const int G = a.group;
  const int32_t* __restrict__ pages = a.kv_indices + a.kv_indptr[it.b];

  // This lane's query row: (token, head) pair r of the group.
  // Rows past the tile's end repeat its last row (every row is computed independently;
  // they are not stored).
  const int r = it.row_begin + 16 * w + n;
  const bool row_valid = r < it.row_end;
  const int re = row_valid ? r : it.row_end - 1;
  const int tok = re / G;
  const int head = kvh * G + re % G;
  const int pos = it.kv_len - it.q_len + tok;
  const int64_t q_row = (int64_t)(it.q_begin + tok) * a.num_qo_heads + head;

  const int kv_lo = it.kv_begin, kv_hi = it.kv_end;
  const int st_first = kv_lo / KS;
  const int st_end = (kv_hi + KS - 1) / KS;

  // Keys row n sees: [vis_lo, vis_lo + vis_len) (the tile's range, the causal bound, the
  // window).
  int vis_lo = kv_lo, vis_hi = kv_hi;
  if (a.causal) vis_hi = min(vis_hi, pos + 1);
  if (a.window > 0) vis_lo = max(vis_lo, pos - a.window + 1);
  const uint32_t vis_len = vis_hi > vis_lo ? (uint32_t)(vis_hi - vis_lo) : 0u;
  const float c = a.scale_log2;

  // Stages [full_lo, full_hi) are visible to every row of this wave without a mask.
  int full_lo, full_hi;
  {
    const int w_row0 = min(it.row_begin + 16 * w, it.row_end - 1);
    const int w_row1 = min(it.row_begin + 16 * w + 15, it.row_end - 1);
    const int p_first = it.kv_len - it.q_len + w_row0 / G;
    const int p_last = it.kv_len - it.q_len + w_row1 / G;
    int hi = kv_hi;                                   // keys < hi are below every bound
    if (a.causal) hi = min(hi, p_first + 1);
    int lo = kv_lo;
    if (a.window > 0) lo = max(lo, p_last - a.window + 1);
    full_lo = (lo + KS - 1) / KS;
    full_hi = hi / KS;
  }

  // Q^T operand for the whole tile: step j holds dims 32j + 8*g4 .. +7 of row n.  Loaded
  // before any stage copy, so waiting for a copy also covers it.
  u32x4_t qf[F8MF ? 1 : QSTEPS];
  // FP8 stages: S^T runs on the FP8 MFMA (16x16x128, see qk), whose B operand holds, in
  // lane (g4, n) at step s, dims 128 s + 32 g4 .. +31 of row n as E4M3 codes.  The 128
  // dims of a (row, step) are scaled by 2^e8 so that their largest magnitude lies in
  // [128, 256), and split into two E4M3 terms, hi = e4m3(q 2^e8) and lo = e4m3(q 2^e8 -
  // hi): their sum is q 2^e8 exactly for every element of at least 1/2 (the top ~9
  // binades), and within 2^-10 of it below.  The MFMA's E8M0 B scale, 2^-e8, undoes the
  // factor.  One exponent per (row, step): the MFMA applies the scale of lane group j to a
  // block of 32 k-slots that spans two lane groups' halves (measured), so the four lane
  // groups of a row carry the same scale.
  constexpr int QS8 = DQK / 128;
  i32x8_t qh[F8MF ? QS8 : 1], ql[F8MF ? QS8 : 1];
  uint32_t qscale = 0;  // E8M0 byte of step s at bits 8 s
  if constexpr (F8MF) {
    const uint16_t* src = a.q + q_row * DQK + 32 * g4;
#pragma unroll
    for (int st8 = 0; st8 < QS8; ++st8) {
      u32x4_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = (*(const u32x4_t*)(src + 128 * st8 + 8 * u) & a.q_and) ^ a.q_xor;
      float mx = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(v[u][e])), fabsf(bf16_hi(v[u][e]))));
      mx = max_xor32(max_xor16(mx));  // the row's four lane groups
      int ex = 0;
      frexpf(mx, &ex);  // mx < 2^ex
      const int e8 = mx > 0.f ? min(max(8 - ex, -127), 127) : 0;
      const float up = __builtin_ldexpf(1.f, e8);
      qscale |= (uint32_t)(127 - e8) << (8 * st8);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float x0 = bf16_lo(v[u][2 * e]) * up, x1 = bf16_hi(v[u][2 * e]) * up;
          const float x2 = bf16_lo(v[u][2 * e + 1]) * up, x3 = bf16_hi(v[u][2 * e + 1]) * up;
          int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
          h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
          const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
          const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
          int l = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - h01[0], x1 - h01[1], 0, false);
          l = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - h23[0], x3 - h23[1], l, true);
          qh[st8][2 * u + e] = h;
          ql[st8][2 * u + e] = l;
        }
      }
    }
  } else {
    // bf16 operands: step j holds dims 32j + 8 g4 .. +7 of row n; FP8 stages widened to
    // bf16 pair the steps instead (see qk): dims 64 (j >> 1) + 16 g4 + 8 (j & 1) .. +7.
    const uint16_t* src = a.q + q_row * DQK + (F8 ? 16 : 8) * g4;
#pragma unroll
    for (int j = 0; j < QSTEPS; ++j)
      qf[j] = *(const u32x4_t*)(src + (F8 ? 64 * (j >> 1) + 8 * (j & 1) : 32 * j));
#pragma unroll
    for (int j = 0; j < QSTEPS; ++j) qf[j] = (qf[j] & a.q_and) ^ a.q_xor;
  }

  // Copies key stage `st` into buffer SLOT.  Wave w moves key rows 4w .. 4w+3 of the stage
  // for both K and V, straight from the pages into LDS (one instruction per 1 KB row, or
  // one per two 512-byte rows); lane L fills chunk position L % chunks-per-row of its row
  // with the logical chunk that the swizzle puts there.  Each instruction takes a
  // wave-uniform 64-bit base and a 32-bit per-lane offset.
  const char* k_base = a.k + (int64_t)kvh * a.k_sh;
  const char* v_base = a.v + (int64_t)kvh * a.v_sh;
  const int my_row = RPW * w;
  // A stage inside one page (page size a multiple of 32): one lookup, then rows at a fixed
  // stride.  The page index and the stage within the page of the next copy are tracked
  // incrementally (copies run in stage order).
  const int stages_per_page = a.page_size / KS;
  int nxt_j = 0, nxt_r = 0;
  uint32_t k_roff = 0, v_roff = 0;  // byte offsets of the next copy's stage inside its page
  if constexpr (PM == kPagesStage) {
    nxt_j = __builtin_amdgcn_readfirstlane(st_first / stages_per_page);
    nxt_r = __builtin_amdgcn_readfirstlane(st_first - nxt_j * stages_per_page);
    k_roff = (uint32_t)nxt_r * KS * (uint32_t)a.k_st;
    v_roff = (uint32_t)nxt_r * KS * (uint32_t)a.v_st;
  }
  // Rows at or past the request's length would read slots past its last page's end (not
  // keys of the request); they re-read the request's last key instead, which sits in the
  // same page.  They are masked out.  The stage base is one 64-bit scalar sum; a row's
  // offset from it fits 32 bits (the host checks that a page's bytes do), so each copy
  // instruction takes a scalar base plus a 32-bit per-lane offset.  copy_prep does the
  // scalar work of a stage once; copy_one issues copy instruction IDX (K rows first, then
  // V rows), so the instructions can be spread over the stage's MFMA steps.  The copies are
  // buffer loads to LDS over a resource at the stage base (the global-memory form would make
  // the compiler drain every LDS read at each later LDS wait, as it counts that form as a
  // pending LDS access).
  constexpr int NKC = RPW / KRPI, NVC = RPW / VRPI, NCOPY = NKC + NVC;
  // The next copy's resources and last in-range row (plain locals, so they stay in
  // scalar registers).  A prep past the last stage (no copy follows it) clamps to the
  // request's last page and row 0 of the stage, so its addresses stay valid.
  __amdgpu_buffer_rsrc_t c_kr = make_rsrc(a.k), c_vr = make_rsrc(a.v);
  int c_last_row = 0;
  const int last_j = (it.kv_len - 1) / a.page_size;
  // Page indices come from a window of 64 consecutive entries held one per lane and read
  // with v_readlane, so a stage's lookup has no memory latency; the window moves (one
  // vector load) every 64 pages.
  int pwin_base = 0, pwin = 0;
  if constexpr (PM == kPagesStage) {
    pwin_base = min(nxt_j, last_j);
    pwin = pages[min(pwin_base + lane, last_j)];
  }
  auto copy_prep = [&](int st) {
    const int jj = min(nxt_j, last_j);
    if (jj - pwin_base >= 64) {
      pwin_base = jj;
      pwin = pages[min(pwin_base + lane, last_j)];
    }
    const int pg = __builtin_amdgcn_readlane(pwin, jj - pwin_base);
    c_last_row = max(it.kv_len - 1 - st * KS, 0);  // a stage that is copied holds a key < kv_len
    // Page strides fit 32 bits on this path (host-checked): one 32x32->64-bit product each.
    c_kr = make_rsrc((const char*)uniform_i64(
        (int64_t)(k_base + (uint64_t)(uint32_t)pg * (uint32_t)a.k_sp + k_roff)));
    c_vr = make_rsrc((const char*)uniform_i64(
        (int64_t)(v_base + (uint64_t)(uint32_t)pg * (uint32_t)a.v_sp + v_roff)));
    k_roff += KS * (uint32_t)a.k_st;
    v_roff += KS * (uint32_t)a.v_st;
    if (++nxt_r == stages_per_page) {
      nxt_r = 0;
      ++nxt_j;
      k_roff = 0;
      v_roff = 0;
    }
  };
  // Instruction IDX % NCOPY of the rows of wave w (IDX < NCOPY) or of wave w + NW/2 (the
  // wave sharing this SIMD, IDX >= NCOPY).
  const uint32_t lane16 = 16u * (uint32_t)lane;
  auto copy_one = [&](auto idx_c, auto slot_c, int vo) {
    constexpr int IDX = decltype(idx_c)::value % NCOPY;
    const int my_row = RPW * w + (decltype(idx_c)::value / NCOPY) * RPW * (NW / 2);
    // One row per instruction: the row is wave-uniform, so its offset goes in the scalar
    // operand and the lane's chunk is 16 lane ^ 16 swizzle (the empty asm hides the swizzle
    // from loop-invariant hoisting, which would hold one register per instruction).
    constexpr bool ONE_ROW = IDX < NKC ? KRPI == 1 : VRPI == 1;
    if constexpr (ONE_ROW) {
      constexpr int i = IDX < NKC ? IDX : IDX - NKC;
      const int row = my_row + i;
      uint32_t sw = 16u * (uint32_t)(IDX < NKC ? k_swz(row) : vswz(row));
      asm volatile("" : "+s"(sw));
      const uint32_t soff = (uint32_t)min(row, c_last_row) * (uint32_t)(IDX < NKC ? a.k_st : a.v_st);
      if constexpr (IDX < NKC)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c_kr,
            (__attribute__((address_space(3))) void*)(k_buf(slot_c) + row * DQK), 16, lane16 ^ sw, soff, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(c_vr,
            (__attribute__((address_space(3))) void*)(v_lds + vo + row * DVO), 16, lane16 ^ sw, soff, 0, 0);
      return;
    }
    // The lane terms are rebuilt from one register each time (the empty asm hides the value
    // from loop-invariant hoisting, which would hold one register per instruction).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if constexpr (IDX < NKC) {
      constexpr int i = IDX * KRPI;
      const int row = my_row + i + (KRPI == 1 ? 0 : (int)((uint32_t)ln / KCH));
      const uint32_t off = (uint32_t)min(row, c_last_row) * (uint32_t)a.k_st +
                           16u * (((uint32_t)ln % KCH) ^ k_swz(row));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c_kr,
          (__attribute__((address_space(3))) void*)(k_buf(slot_c) + (my_row + i) * DQK), 16, off, 0, 0, 0);
    } else {
      constexpr int i = (IDX - NKC) * VRPI;
      const int row = my_row + i + (VRPI == 1 ? 0 : (int)((uint32_t)ln / VCH));
      const uint32_t off = (uint32_t)min(row, c_last_row) * (uint32_t)a.v_st +
                           16u * (((uint32_t)ln % VCH) ^ vswz(row));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c_vr,
          (__attribute__((address_space(3))) void*)(v_lds + vo + (my_row + i) * DVO), 16, off, 0, 0, 0);
    }
  };
  // NVFP4 (converted on the way in): lane l holds key row my_row + l / 16 of the stage
  // and, of its K and V rows, the 8-element chunks c = l % 16 + 16 k (k < D / 128), so that
  // each store instruction writes 16 consecutive chunk positions of a row (a
  // bank-conflict-free 256 bytes; chunks strided by four positions per lane conflicted in
  // 4-way groups).  Key rows are clamped into the tile's range like the copies' (clamped
  // keys are masked out).
  constexpr int KC = DQK / 128, VC = DVO / 128;  // chunks per lane and row
  // Byte address of row t's K and V rows (and block-scale rows) in the pages.
  auto conv_rows = [&](int st, const char*& kd, const char*& vd, const char*& ks, const char*& vs) {
    if constexpr (PM == kPagesStage) {
      // The stage lies in one page: one lookup, tracked in stage order like the copies'
      // (stages are loaded in order), and rows at fixed strides.  Rows at or past the
      // request's length re-read its last key (same page; masked out).
      const int jj = min(nxt_j, last_j);
      if (jj - pwin_base >= 64) {
        pwin_base = jj;
        pwin = pages[min(pwin_base + lane, last_j)];
      }
      const int64_t pg = __builtin_amdgcn_readlane(pwin, jj - pwin_base);
      const int row = min(my_row + (lane >> 4), max(it.kv_len - 1 - st * KS, 0));
      const int64_t sl = (int64_t)nxt_r * KS + row;
      kd = a.k + pg * a.k_sp + (int64_t)kvh * a.k_sh + sl * a.k_st;
      vd = a.v + pg * a.v_sp + (int64_t)kvh * a.v_sh + sl * a.v_st;
      ks = a.k_sf + pg * a.ks_sp + (int64_t)kvh * a.ks_sh + sl * a.ks_st;
      vs = a.v_sf + pg * a.vs_sp + (int64_t)kvh * a.vs_sh + sl * a.vs_st;
      if (++nxt_r == stages_per_page) {
        nxt_r = 0;
        ++nxt_j;
      }
      return;
    }
    int t = st * KS + my_row + (lane >> 4);
    t = t < kv_lo ? kv_lo : (t >= kv_hi ? kv_hi - 1 : t);
    const int j = t / a.page_size;
    const int64_t pg = pages[j];
    const int64_t sl = t - j * a.page_size;
    kd = a.k + pg * a.k_sp + (int64_t)kvh * a.k_sh + sl * a.k_st;
    vd = a.v + pg * a.v_sp + (int64_t)kvh * a.v_sh + sl * a.v_st;
    if constexpr (FP4) {
      ks = a.k_sf + pg * a.ks_sp + (int64_t)kvh * a.ks_sh + sl * a.ks_st;
      vs = a.v_sf + pg * a.vs_sp + (int64_t)kvh * a.vs_sh + sl * a.vs_st;
    }
  };
  // NVFP4: chunk c is 4 packed bytes at 4 c; its block scale is byte c / 2 of the row's
  // scales (one E4M3 code per 16 elements).
  uint32_t fk[KC], fv[VC], fks[KC], fvs[VC];
  auto fp4_load = [&](int st) {
    const int part = lane & 15;
    const char *kd, *vd, *ks, *vs;
    conv_rows(st, kd, vd, ks, vs);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      fk[k] = *(const uint32_t*)(kd + 4 * (part + 16 * k));
      fks[k] = *(const uint8_t*)(ks + ((part + 16 * k) >> 1));
    }
#pragma unroll
    for (int k = 0; k < VC; ++k) {
      fv[k] = *(const uint32_t*)(vd + 4 * (part + 16 * k));
      fvs[k] = *(const uint8_t*)(vs + ((part + 16 * k) >> 1));
    }
  };
  // Converts the loaded chunks (e2m1 x block scale, exact in bf16) and writes chunk c at
  // position c ^ swizzle(row).
  auto fp4_store = [&](auto slot_c, int vo) {
    const int row = my_row + (lane >> 4);
    const int part = lane & 15;
    auto chunk8 = [&](uint32_t w, float bs) {
      float e[8];
      fp4x8_to_f32(w, e);
      u32x4_t pk;
#pragma unroll
      for (int u = 0; u < 4; ++u) pk[u] = pack_bf16(e[2 * u] * bs, e[2 * u + 1] * bs);
      return pk;
    };
    st_t* kd = k_buf(slot_c) + row * DQK;
#pragma unroll
    for (int k = 0; k < KC; ++k)
      *(u32x4_t*)(kd + 8 * ((part + 16 * k) ^ k_swz(row))) = chunk8(fk[k], fp8_to_f32<0>(fks[k]));
    st_t* vd = v_lds + vo + row * DVO;
#pragma unroll
    for (int k = 0; k < VC; ++k)
      *(u32x4_t*)(vd + 8 * ((part + 16 * k) ^ v_swz(row))) = chunk8(fv[k], fp8_to_f32<0>(fvs[k]));
    // The writes complete before this wave reaches the barrier that hands the stage over.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  };

  auto conv_store = [&](auto slot_c, int vo) { fp4_store(slot_c, vo); };

  // Copies stage st: K into buffer slot_c, V into v_lds + vo (converting formats: loads the
  // codes into registers; conv_store then writes them).
  auto copy_stage = [&](int st, auto slot_c, int vo) {
    if constexpr (FP4) {
      fp4_load(st);
    } else if constexpr (PM == kPagesStage) {
      copy_prep(st);
      static_for<NCOPY>([&](auto idx_c) { copy_one(idx_c, slot_c, vo); });
    } else {
      // One page-table lookup per key row (keys clamped into the tile's range, so every
      // row read is a key of the request; clamped keys are masked out).
      auto row_base = [&](int row, const char* base, int64_t sp, int64_t stt) {
        int t = st * KS + my_row + row;
        t = t < kv_lo ? kv_lo : (t >= kv_hi ? kv_hi - 1 : t);
        int pg, sl;
        uniform_page_slot<PM == kPagesPow2>(pages, t, a.page_size, a.page_shift, pg, sl);
        return (const char*)uniform_i64((int64_t)(base + pg * sp + sl * stt));
      };
      int ln = lane;
      asm volatile("" : "+v"(ln));
      // Row base of lane sub-row `sub` when one instruction covers RPI rows.
      auto sub_base = [&](auto rpi_c, int i, uint32_t sub, const char* base, int64_t sp, int64_t stt) {
        constexpr int RPI = decltype(rpi_c)::value;
        const char* rb = row_base(i, base, sp, stt);
#pragma unroll
        for (int u = 1; u < RPI; ++u) {
          const char* ru = row_base(i + u, base, sp, stt);
          rb = sub == (uint32_t)u ? ru : rb;
        }
        return rb;
      };
#pragma unroll
      for (int i = 0; i < RPW; i += KRPI) {
        const uint32_t sub = KRPI == 1 ? 0u : (uint32_t)ln / KCH;
        const char* rb = sub_base(std::integral_constant<int, KRPI>{}, i, sub, k_base, a.k_sp, a.k_st);
        const uint32_t off = 16u * (((uint32_t)ln % KCH) ^ k_swz(my_row + i + (int)sub));
        __builtin_amdgcn_global_load_lds((const void*)(rb + off),
            (__attribute__((address_space(3))) void*)(k_buf(slot_c) + (my_row + i) * DQK), 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < RPW; i += VRPI) {
        const uint32_t sub = VRPI == 1 ? 0u : (uint32_t)ln / VCH;
        const char* rb = sub_base(std::integral_constant<int, VRPI>{}, i, sub, v_base, a.v_sp, a.v_st);
        const uint32_t off = 16u * (((uint32_t)ln % VCH) ^ vswz(my_row + i + (int)sub));
        __builtin_amdgcn_global_load_lds((const void*)(rb + off),
            (__attribute__((address_space(3))) void*)(v_lds + vo + (my_row + i) * DVO), 16, 0, 0);
      }
    }
  };

  f32x4_t o[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref = -INFINITY;  // reference max of row n (log2 domain)
  float l_run = 0.f;        // this lane's share of the row sum
  float l_bf = 0.f;         // the same over the bf16-rounded weights

  // One-lookup pages: the first wave group issues all of the next stage's copies (its rows
  // and its SIMD partner's), one per S^T step, so the vector memory pipe streams them while
  // the MFMAs run; the second group issues none (as bursts at the interval start they stall
  // the issuing waves).  Other page sizes: every wave copies its own rows at the interval
  // start.
  constexpr bool SPREAD = PM == kPagesStage && !CONV;
  // NVFP4 holds a stage's codes in registers, which the 512/512 form has no room for: the
  // host runs NVFP4 at 512/512 as two 512/256 launches, one per half of the value head_dim.
  static_assert(!(CONV && DQK == 512 && DVO == 512), "NVFP4 at 512/512 runs as two 512/256 halves");
  // ---- S^T = K Q^T from K buffer kslot_c into s0 (keys 0..15) and s1 (keys 16..31); lane
  // holds keys 4*g4 + i.  With COPY the next stage's copies (K into the other buffer, V into
  // v_lds + vo_next) are issued among the steps.
  f32x4_t s0, s1;
  auto qk = [&](auto kslot_c, auto copy_c, int vo_next) {
    constexpr bool COPY = decltype(copy_c)::value;
    const st_t* kt = k_buf(kslot_c);
    s0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    s1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // With COPY this wave issues the copies of its own rows and of its SIMD partner's.
    constexpr int NQC = 2 * NCOPY;
    constexpr int CSTEP = QSTEPS / NQC > 0 ? QSTEPS / NQC : 1;
    static_assert(!COPY || (QSTEPS + CSTEP - 1) / CSTEP >= NQC, "copy slots");
    if constexpr (F8MF) {
      // v_mfma_scale_f32_16x16x128_f8f6f4 on the codes as they are: step s contracts over
      // dims 128 s .. +127, lane (g4, n) holding dims 128 s + 32 g4 .. +31 of key row n (A)
      // and the query's hi and lo terms (B; one MFMA each, measured: A's lane/byte k-slot
      // pairs with B's at the same lane group and byte).  The 32 codes are chunks 8s + 2 g4
      // and 8s + 2 g4 + 1 of the row, at positions (8s + 2 g4 + h) ^ n, i.e.
      // 8 (s ^ (n >> 3)) + ((2 g4 + h) ^ (n & 7)): with bit 7 of kb holding n >> 3 (DQK 256:
      // s < 2) and bit 4 the low bit of (2 g4) ^ (n & 7), the reads are at kb ^ 128 s and
      // kb ^ 16 ^ 128 s.
      constexpr int CPS = (NQC + QS8 - 1) / QS8;  // copies issued per step
      int kb = n * DQK + 128 * (n >> 3) + 16 * ((2 * g4) ^ (n & 7));
      asm volatile("" : "+v"(kb));
      // Key rows n (tile 0) and 16 + n (tile 1): one operand buffer each, refilled with the
      // next step's codes right after the two MFMAs that read it.
      auto ld = [&](int st8, int tile) {
        const st_t* p0 = kt + (kb ^ (128 * st8)) + 16 * DQK * tile;
        const st_t* p1 = kt + ((kb ^ 16) ^ (128 * st8)) + 16 * DQK * tile;
        const u32x4_t a0 = *(const u32x4_t*)p0, a1 = *(const u32x4_t*)p1;
        return i32x8_t{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
      };
      i32x8_t k0 = ld(0, 0), k1 = ld(0, 1);
      static_for<QS8>([&](auto s_c) {
        constexpr int st8 = decltype(s_c)::value;
        if constexpr (COPY) {
          static_for<CPS>([&](auto u_c) {
            constexpr int ci = st8 * CPS + decltype(u_c)::value;
            if constexpr (ci < NQC)
              copy_one(std::integral_constant<int, ci>{},
                       std::integral_constant<int, decltype(kslot_c)::value ^ 1>{}, vo_next);
          });
        }
        constexpr int sa = 0x7F7F7F7F;  // E8M0 1.0 for the codes
        s0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k0, qh[st8], s0, 0, 0, 0, sa, st8, (int)qscale);
        s0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k0, ql[st8], s0, 0, 0, 0, sa, st8, (int)qscale);
        s1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k1, qh[st8], s1, 0, 0, 0, sa, st8, (int)qscale);
        s1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k1, ql[st8], s1, 0, 0, 0, sa, st8, (int)qscale);
        if constexpr (st8 + 1 < QS8) {
          k0 = ld(st8 + 1, 0);
          k1 = ld(st8 + 1, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      return;
    }
    if constexpr (F8) {
      // K widened to bf16 after the read.  The contraction order over head_dim is free as
      // long as K and Q agree: steps 2p and 2p + 1 take lane group g4's dims 64p + 16 g4 ..
      // +15, so one 16-byte read of key row n (and 16 + n) serves both (codes 0-7, then
      // 8-15).  That chunk, 4p + g4, sits at position (4p + g4) ^ n; bits 6-7 of kb hold
      // n >> 2 and nothing else, so pair p's byte offset is kb ^ 64 (p & 3), plus 256 (p >> 2).
      constexpr int KP = 2;  // pairs read ahead
      int kb = n * DQK + 16 * (g4 ^ (n & 3)) + 64 * (n >> 2);
      asm volatile("" : "+v"(kb));
      auto ld = [&](int p, u32x4_t& k0, u32x4_t& k1) {
        const st_t* src = kt + ((kb ^ (64 * (p & 3))) + 256 * (p >> 2));
        k0 = *(const u32x4_t*)src;
        k1 = *(const u32x4_t*)(src + 16 * DQK);
      };
      u32x4_t kr0[KP + 1], kr1[KP + 1];
#pragma unroll
      for (int p = 0; p < KP; ++p) ld(p, kr0[p], kr1[p]);
      static_for<QSTEPS>([&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        constexpr int p = j >> 1, r = p % (KP + 1);
        if constexpr ((j & 1) == 0 && p + KP < QSTEPS / 2)
          ld(p + KP, kr0[(p + KP) % (KP + 1)], kr1[(p + KP) % (KP + 1)]);
        if constexpr (COPY && j % CSTEP == 0 && j / CSTEP < NQC)
          copy_one(std::integral_constant<int, j / CSTEP>{},
                   std::integral_constant<int, decltype(kslot_c)::value ^ 1>{}, vo_next);
        const bf16x8_t qb = __builtin_bit_cast(bf16x8_t, qf[j]);
        const u32x2_t c0 = {kr0[r][2 * (j & 1)], kr0[r][2 * (j & 1) + 1]};
        const u32x2_t c1 = {kr1[r][2 * (j & 1)], kr1[r][2 * (j & 1) + 1]};
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(c0), qb, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(c1), qb, s1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
      return;
    }
    // Element index of the step-j chunk: kb ^ 32*(j & 3) (bits 5-6 of kb hold n >> 2 and
    // nothing else does), plus 128*(j >> 2).
    int kb = n * DQK + 8 * (g4 ^ (n & 3)) + 32 * (n >> 2);
    asm volatile("" : "+v"(kb));
    // Tile 1's row is read first: the wait for tile 0's read then covers both, so the two
    // MFMAs of a step follow one wait.
    auto ld = [&](int j, u32x4_t& k0, u32x4_t& k1) {
      const st_t* src = kt + ((kb ^ (32 * (j & 3))) + 128 * (j >> 2));
      k1 = *(const u32x4_t*)(src + 16 * DQK);
      k0 = *(const u32x4_t*)src;
    };
    u32x4_t kr0[KD + 1], kr1[KD + 1];
#pragma unroll
    for (int j = 0; j < KD; ++j) ld(j, kr0[j], kr1[j]);
    static_for<QSTEPS>([&](auto j_c) {
      constexpr int j = decltype(j_c)::value;
      if constexpr (j + KD < QSTEPS) ld(j + KD, kr0[(j + KD) % (KD + 1)], kr1[(j + KD) % (KD + 1)]);
      if constexpr (COPY && j % CSTEP == 0 && j / CSTEP < NQC)
        copy_one(std::integral_constant<int, j / CSTEP>{},
                 std::integral_constant<int, decltype(kslot_c)::value ^ 1>{}, vo_next);
      const bf16x8_t qb = __builtin_bit_cast(bf16x8_t, qf[j]);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr0[j % (KD + 1)]), qb, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr1[j % (KD + 1)]), qb, s1, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- online softmax of stage stp's scores (s0, s1) into the P^T operand pf, with the
  // lazy rescale of the running state.
  u32x4_t pf;
  // Masks and online softmax of row n (its 32 keys are spread over the 4 lanes g4).  The
  // scale is positive: masks and the max work on raw scores, and the scale folds into one
  // FMA per key in the exponent.
  auto softmax = [&](int stp) {
    const int t0 = stp * KS;
    const bool full = stp >= full_lo && stp < full_hi;
    float sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = i < 4 ? s0[i] : s1[i - 4];
    if (!full) {
      // Key t is visible to row n iff t - vis_lo < vis_len (unsigned): one compare a key.
      const uint32_t base = (uint32_t)(t0 + 4 * g4 - vis_lo);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool ok = base + (uint32_t)(16 * (i >> 2) + (i & 3)) < vis_len;
        sv[i] = ok ? sv[i] : -INFINITY;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    mx = max_xor16(mx);
    mx = max_xor32(mx) * c;
    // Move the reference max only when the row max outgrows it by the threshold.  While
    // m_ref is -inf (no visible key yet) any finite max outgrows it, and the factor
    // exp2(-inf) = 0 clears the (zero) state.
    const bool grow = mx > m_ref + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mx : m_ref;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
      l_run *= alpha;
      l_bf *= alpha;
#pragma unroll
      for (int t = 0; t < OT; ++t) o[t] *= alpha;
      m_ref = m_new;
    }
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    // P^T operand: k-slot e of lane group g4 is key 4*g4 + e (e < 4) or 16 + 4*g4 + e - 4.
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(fmaf(sv[i], c, -m_use));
      l_run += p[i];
    }
    // The output is normalised by the sum of the bf16 weights the MFMA uses, so the applied
    // weights sum to one (this matters when one key dominates the row); the lse uses the
    // fp32 sum.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pf[e] = pack_bf16(p[2 * e], p[2 * e + 1]);
      l_bf += bf16_lo(pf[e]) + bf16_hi(pf[e]);
    }
  };

  // ---- O^T += V^T P^T from the V buffer at v_lds + vo.  A operand of lane (g4, m=n):
  // V[k-slot keys][dim 16t + m], from two transpose reads (keys 4*g4 + 0..3 and
  // 16 + 4*g4 + 0..3; both rows have the same swizzle, and the second is 16 rows below the
  // first).  Software-pipelined like S^T: tile t + VD's reads are issued before tile t's
  // MFMA.  The reads are inline assembly (see lds_read_tr16_at), so each MFMA first waits
  // for its own tile's two reads: at most 2 * (tiles issued after it) reads may be pending.
  // Transpose-read source of this lane within its 16-lane block: key (n / 4) of the 4-key
  // group, dims 4*(n % 4) .. +3 of the 16-dim tile.  Byte address of tile t's chunk:
  // vb ^ 32*(t & 7) (bits 5-7 of vb hold the row swizzle and nothing else does), plus
  // 256*(t >> 3) as the instruction offset.
  const int tr_row = 4 * g4 + (n >> 2);
  const uint32_t vb_lane =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint16_t*)(
          v_lds + tr_row * DVO + 4 * (n & 1) + 8 * ((n & 3) >> 1)) +
      32u * (uint32_t)(tr_row & 7);
  // FP8 stages: the A operand's k-slots follow P's, keys 4 g4 + 0..3 then 16 + 4 g4 + 0..3.
  // Lane (g4, n) of a transpose read addresses the key row of k-slot n >> 1, half n & 1 of
  // tile t's chunk (the 16 codes of dims 16t .. 16t + 15), at chunk position t ^ swizzle;
  // it receives dim 16t + n of the eight k-slot keys: one read per tile gives the eight
  // codes of the A operand.  Bits 4-7 of vb8_lane hold the swizzle and nothing else, so
  // tile t's address is vb8_lane ^ 16 (t & 15), plus 256 (t >> 4) as the instruction offset.
  const int tr8_row = 4 * g4 + ((n >> 1) & 3) + 16 * (n >> 3);
  const uint32_t vb8_lane =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const st_t*)(
          v_lds + tr8_row * DVO + (F8 ? 8 * (n & 1) : 0)) +
      16u * (uint32_t)v_swz_fp8(tr8_row);
  auto pv = [&](int vo) {
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pf);
    if constexpr (F8) {
      uint32_t vb = vb8_lane + (uint32_t)vo;
      asm volatile("" : "+v"(vb));
      u32x2_t vr[VD + 1];
      auto ld = [&](auto t_c) {
        constexpr int t = decltype(t_c)::value;
        vr[t % (VD + 1)] = lds_read_tr8_at<256 * (t >> 4)>(vb ^ (16u * (t & 15)));
      };
      static_for<VD>([&](auto t_c) { ld(t_c); });
      static_for<OT>([&](auto t_c) {
        constexpr int t = decltype(t_c)::value;
        constexpr int r = t % (VD + 1);
        if constexpr (t + VD < OT) ld(std::integral_constant<int, t + VD>{});
        lds_wait<(t + VD < OT ? VD : OT - 1 - t)>(vr[r]);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(vr[r]), pb, o[t], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
      return;
    }
    uint32_t vb = vb_lane + 2u * (uint32_t)vo;
    asm volatile("" : "+v"(vb));
    u32x2_t vlo[VD + 1], vhi[VD + 1];
    auto ld = [&](auto t_c) {
      constexpr int t = decltype(t_c)::value;
      const uint32_t src = vb ^ (32u * (t & 7));
      vlo[t % (VD + 1)] = lds_read_tr16_at<256 * (t >> 3)>(src);
      vhi[t % (VD + 1)] = lds_read_tr16_at<256 * (t >> 3) + 32 * DVO>(src);
    };
    static_for<VD>([&](auto t_c) { ld(t_c); });
    static_for<OT>([&](auto t_c) {
      constexpr int t = decltype(t_c)::value;
      constexpr int r = t % (VD + 1);
      // Wait for tile t's reads before issuing tile t + VD's: those reads then separate the
      // wait (which the compiler takes as writing the operand registers) from the MFMA, in
      // place of a wait state.
      lds_wait<2 * (t + VD - 1 < OT ? VD - 1 : OT - 1 - t)>(vlo[r], vhi[r]);
      if constexpr (t + VD < OT) ld(std::integral_constant<int, t + VD>{});
      const u32x4_t vf = {vlo[r][0], vlo[r][1], vhi[r][0], vhi[r][1]};
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vf), pb, o[t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- the stage loop, one interval per stage.  Stage st's K sits in K buffer
  // (st - st_first) % 2, its V at v_lds + (st - st_first) % 3 * VSTAGE.  Interval st waits
  // for stage st's copies and meets the other waves at the barrier, then copies stage
  // st + 1.  The two waves sharing a SIMD (w and w + 4) work in rotated order, so that one's
  // softmax runs while the other's MFMAs do: the first group does S^T(st), softmax(st) and
  // O += V P^T(st); the second does softmax(st - 1) and O += V P^T(st - 1) (with stage st -
  // 1's scores kept from the previous interval), then S^T(st), and after the last interval
  // the last stage's softmax and O update.  After barrier st every wave is done with stage
  // st - 1's K buffer (read in interval st - 1 by both groups) and with stage st - 2's V
  // buffer (read in interval st - 2 by the first group and st - 1 by the second), which the
  // copies of stage st + 1 refill.
  const bool second = w >= NW / 2;
  int vo_prev = 2 * VSTAGE, vo_cur = 0, vo_next = VSTAGE;
  if (st_first < st_end) {
    copy_stage(st_first, std::integral_constant<int, 0>{}, 0);
    if constexpr (CONV) conv_store(std::integral_constant<int, 0>{}, 0);
  }
  auto interval = [&](int st, auto kslot_c, auto second_c) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    const bool has_next = st + 1 < st_end;
    constexpr auto other_c = std::integral_constant<int, decltype(kslot_c)::value ^ 1>{};
    if constexpr (decltype(second_c)::value) {
      if (!SPREAD && has_next) copy_stage(st + 1, other_c, vo_next);
      if (st > st_first) {
        softmax(st - 1);
        pv(vo_prev);
      }
      qk(kslot_c, std::false_type{}, vo_next);
    } else {
      if constexpr (SPREAD) {
        if (has_next) {
          copy_prep(st + 1);
          qk(kslot_c, std::true_type{}, vo_next);
        } else {
          qk(kslot_c, std::false_type{}, vo_next);
        }
      } else {
        if (has_next) copy_stage(st + 1, other_c, vo_next);
        qk(kslot_c, std::false_type{}, vo_next);
      }
      softmax(st);
      pv(vo_cur);
    }
    if constexpr (CONV) {
      if (has_next) conv_store(other_c, vo_next);
    }
    const int t = vo_prev;
    vo_prev = vo_cur;
    vo_cur = vo_next;
    vo_next = t;
  };
  // Separate loops per group (one loop holding both orders made the register allocator
  // spill); both meet the same barriers, one per interval.
  auto run = [&](auto second_c) {
    for (int st = st_first; st < st_end; st += 2) {
      interval(st, std::integral_constant<int, 0>{}, second_c);
      if (st + 1 < st_end) interval(st + 1, std::integral_constant<int, 1>{}, second_c);
    }
    if constexpr (decltype(second_c)::value) {
      if (st_first < st_end) {
        softmax(st_end - 1);
        pv(vo_prev);
      }
    }
  };
  // SHORT form: a wave whose 16 rows all lie past the tile's end (a tile of a few new
  // tokens, a request's last tile) computes nothing: it only moves its share of each next
  // stage and meets the same barriers.
  auto idle_interval = [&](int st, auto kslot_c) {
    wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    constexpr auto other_c = std::integral_constant<int, decltype(kslot_c)::value ^ 1>{};
    if (st + 1 < st_end) {
      if constexpr (SPREAD) {
        if (!second) {
          copy_prep(st + 1);
          static_for<2 * NCOPY>([&](auto idx_c) { copy_one(idx_c, other_c, vo_next); });
        }
      } else {
        copy_stage(st + 1, other_c, vo_next);
        if constexpr (CONV) conv_store(other_c, vo_next);
      }
    }
    const int t = vo_prev;
    vo_prev = vo_cur;
    vo_cur = vo_next;
    vo_next = t;
  };
  if constexpr (SHORT) {
    if (it.row_begin + 16 * w >= it.row_end) {  // wave-uniform
      for (int st = st_first; st < st_end; st += 2) {
        idle_interval(st, std::integral_constant<int, 0>{});
        if (st + 1 < st_end) idle_interval(st + 1, std::integral_constant<int, 1>{});
      }
      return;
    }
  }
  if (second) run(std::true_type{});
  else run(std::false_type{});

  // ---- normalise and write row n: O^T tile t, register i holds dim 16t + 4*g4 + i.
  const float l_tot = sum_xor32(sum_xor16(l_run));
  const float l_bf_tot = sum_xor32(sum_xor16(l_bf));
  if (!row_valid) return;
  float inv = l_bf_tot > 0.f ? 1.f / l_bf_tot : 0.f;
  inv *= a.v_scale;  // 1 for a bf16 cache
  if (it.slot >= 0) {
    // One key chunk of a split tile: its normalised output and two log-sum-exps, over the
    // bf16-rounded weights (the merge weights, so the merged output is normalised by the
    // whole bf16 sum as an unsplit tile is) and over the fp32 weights (the lse).
    const int64_t prow = ((int64_t)it.slot * hkv + kvh) * kPrefillTileRows + (r - it.row_begin);
    float* po = a.part_o + prow * DVO;
#pragma unroll
    for (int t = 0; t < OT; ++t) *(f32x4_t*)(po + 16 * t + 4 * g4) = o[t] * inv;
    if (g4 == 0) {
      a.part_lse[2 * prow] = l_bf_tot > 0.f ? m_ref + log2f(l_bf_tot) : -INFINITY;
      a.part_lse[2 * prow + 1] = l_tot > 0.f ? m_ref + log2f(l_tot) : -INFINITY;
    }
    return;
  }
  const int64_t out_row = q_row * a.out_stride;
#pragma unroll
  for (int t = 0; t < OT; ++t) {
    const int d = 16 * t + 4 * g4;
    const f32x4_t v = o[t] * inv;
    if (a.out_fp32) {
      *(f32x4_t*)((float*)a.out + out_row + d) = v;
    } else {
      *(u32x2_t*)((uint16_t*)a.out + out_row + d) = u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    }
  }
  if (a.lse && g4 == 0)
    a.lse[q_row] = l_tot > 0.f ? (m_ref + log2f(l_tot)) * kLn2 : -INFINITY;
}

// Widening of NVFP4 pages for prefill (the NVFP4 page's block format: E2M1 pairs, one E4M3
// scale per 16 elements): page-table entry j's K and V rows become bf16 rows of staged page
// j (each value times its block scale, exact in bf16), and entry j of `ident` becomes j, so
// the bf16 kernel reads staged page j where the table lists page kv_indices[j].
struct StageArgs {
  const char* k;
  const char* v;
  const char* k_sf;
  const char* v_sf;
  int64_t k_sp, k_sh, k_st, v_sp, v_sh, v_st;        // data strides, bytes
  int64_t ks_sp, ks_sh, ks_st, vs_sp, vs_sh, vs_st;  // block-scale strides, bytes
  const int32_t* kv_indices;
  uint16_t* k_out;  // [entry][kv head][slot][head_dim_qk] bf16
  uint16_t* v_out;  // [entry][kv head][slot][head_dim_vo] bf16
  int32_t* ident;
  int32_t num_kv_heads, page_size, dqk, dvo;
};

// One page of one head: `rows` rows of D elements; each thread widens 8 elements (one
// 4-byte word of codes) at a time.
__device__ __forceinline__ void stage_rows(const char* src, int64_t st, const char* sf,
                                           int64_t sst, uint16_t* dst, int D, int rows) {
  const int words = D / 8;
  for (int i = threadIdx.x; i < rows * words; i += blockDim.x) {
    const int r = i / words, w = i - r * words;
    const uint32_t codes = *(const uint32_t*)(src + r * st + 4 * w);
    const uint32_t sbyte = *(const uint8_t*)(sf + r * sst + (w >> 1));
    float scale[4];
    fp8x4_to_f32(sbyte, scale);
    float f[8];
    fp4x8_to_f32(codes, f);
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // products of a 2-bit and a 4-bit significand: exact in bf16, so truncation is exact
      const uint32_t lo = __float_as_uint(f[2 * e] * scale[0]) >> 16;
      const uint32_t hi = __float_as_uint(f[2 * e + 1] * scale[0]) >> 16;
      o[e] = lo | (hi << 16);
    }
    *(u32x4_t*)(dst + (int64_t)r * D + 8 * w) = o;
  }
}

__global__ __launch_bounds__(256) void nvfp4_stage_kernel(StageArgs a) {
  const int64_t j = blockIdx.x;
  const int h = blockIdx.y;
  const int64_t page = a.kv_indices[j];
  if (h == 0 && threadIdx.x == 0) a.ident[j] = (int32_t)j;
  const int64_t slab = (j * a.num_kv_heads + h) * a.page_size;
  stage_rows(a.k + page * a.k_sp + h * a.k_sh, a.k_st, a.k_sf + page * a.ks_sp + h * a.ks_sh,
             a.ks_st, a.k_out + slab * a.dqk, a.dqk, a.page_size);
  stage_rows(a.v + page * a.v_sp + h * a.v_sh, a.v_st, a.v_sf + page * a.vs_sp + h * a.vs_sh,
             a.vs_st, a.v_out + slab * a.dvo, a.dvo, a.page_size);
}

struct PrefillMergeArgs {
  const PrefillMerge* merges;
  const float* part_o;
  const float* part_lse;
  void* out;
  int32_t out_stride;
  float* lse;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t out_fp32;
};

// Split tiles: one wave per (tile, KV head, row); workgroups of 4 waves take 4 consecutive
// rows (grid: merges x KV heads x tile_rows / 4).  The chunk outputs are weighted by
// exp2(lse_bf(c) - max) / sum (chunks with no visible key have lse -inf and weight 0); the
// lse is the log-sum-exp of the fp32 ones.  A row with no visible key at all gets a zero
// output and lse -inf.  Lane l owns dims DVO/64 * l .. +DVO/64.  The chunks' log-sum-exps
// are read one per lane, 64 chunks a pass, and UN chunk rows are requested at once; every
// row is added in chunk order.
template <int DVO>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillMergeArgs a) {
  constexpr int E = DVO / 64;
  constexpr int UN = 8;  // chunk rows in flight
  const PrefillMerge m = a.merges[blockIdx.x];
  const int kvh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int rr = 4 * blockIdx.z + (threadIdx.x >> 6);
  if (rr >= m.row_end - m.row_begin) return;
  const int r = m.row_begin + rr;
  const int tok = r / a.group, head = kvh * a.group + r % a.group;
  const int64_t q_row = (int64_t)(m.q_begin + tok) * a.num_qo_heads + head;
  const int64_t row0 = ((int64_t)m.slot_begin * a.num_kv_heads + kvh) * kPrefillTileRows + rr;
  const int64_t step = (int64_t)a.num_kv_heads * kPrefillTileRows;  // rows between slots
  const int n = m.num_slots;
  auto lse_of = [&](int c) { return *(const f32x2_t*)(a.part_lse + 2 * (row0 + c * step)); };
  float mw = -INFINITY, mo = -INFINITY;
  for (int c0 = 0; c0 < n; c0 += 64) {
    if (c0 + lane < n) {
      const f32x2_t l = lse_of(c0 + lane);
      mw = fmaxf(mw, l[0]);
      mo = fmaxf(mo, l[1]);
    }
  }
  mw = max_xor16(max_xor32(mw));
  mo = max_xor16(max_xor32(mo));
#pragma unroll
  for (int s = 8; s >= 1; s >>= 1) {
    mw = fmaxf(mw, shfl_xor_f(mw, s));
    mo = fmaxf(mo, shfl_xor_f(mo, s));
  }
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float sw = 0.f, so = 0.f;  // this lane's chunks
  const float* src0 = a.part_o + row0 * DVO + E * lane;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int cn = min(64, n - c0);
    float w = 0.f;
    if (lane < cn) {
      const f32x2_t l = lse_of(c0 + lane);
      w = l[0] == -INFINITY ? 0.f : exp2f(l[0] - mw);
      so += l[1] == -INFINITY ? 0.f : exp2f(l[1] - mo);
      sw += w;
    }
    for (int c = 0; c < cn; c += UN) {
      f32x4_t x[UN][E / 4];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int cc = c0 + min(c + u, cn - 1);  // past the end: the last chunk, weight 0
#pragma unroll
        for (int e = 0; e < E / 4; ++e) x[u][e] = *(const f32x4_t*)(src0 + cc * step * DVO + 4 * e);
      }
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), c + u));
#pragma unroll
        for (int e = 0; e < E / 4; ++e)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[4 * e + v] = fmaf(wu, x[u][e][v], acc[4 * e + v]);
      }
    }
  }
  sw = sum_xor16(sum_xor32(sw));
  so = sum_xor16(sum_xor32(so));
#pragma unroll
  for (int s = 8; s >= 1; s >>= 1) {
    sw += shfl_xor_f(sw, s);
    so += shfl_xor_f(so, s);
  }
  const float inv = sw > 0.f ? 1.f / sw : 0.f;
  const int64_t off = q_row * a.out_stride + E * lane;
#pragma unroll
  for (int e = 0; e < E; e += 4) {
    const f32x4_t v = {acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv};
    if (a.out_fp32) *(f32x4_t*)((float*)a.out + off + e) = v;
    else *(u32x2_t*)((uint16_t*)a.out + off + e) = u32x2_t{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  }
  if (a.lse && lane == 0) a.lse[q_row] = so > 0.f ? (mo + log2f(so)) * kLn2 : -INFINITY;
}

template <int DQK, int DVO, bool SHORT>
static void launch_prefill(const PrefillArgs& a, int pm, int kv, int grid, hipStream_t s) {
  if (kv == kKvFp4) {
    if constexpr (!(DQK == 512 && DVO == 512)) {  // 512/512 runs as two 512/256 halves
      if (pm == kPagesStage) prefill_kernel<DQK, DVO, kPagesStage, kKvFp4, SHORT><<<grid, 512, 0, s>>>(a);
      else prefill_kernel<DQK, DVO, kPagesAny, kKvFp4, SHORT><<<grid, 512, 0, s>>>(a);
    }
  } else if (kv == kKvFp8) {
    if (pm == kPagesStage) prefill_kernel<DQK, DVO, kPagesStage, kKvFp8, SHORT><<<grid, 512, 0, s>>>(a);
    else if (pm == kPagesPow2) prefill_kernel<DQK, DVO, kPagesPow2, kKvFp8, SHORT><<<grid, 512, 0, s>>>(a);
    else prefill_kernel<DQK, DVO, kPagesAny, kKvFp8, SHORT><<<grid, 512, 0, s>>>(a);
  } else if (pm == kPagesStage) prefill_kernel<DQK, DVO, kPagesStage, kKvBf16, SHORT><<<grid, 512, 0, s>>>(a);
  else if (pm == kPagesPow2) prefill_kernel<DQK, DVO, kPagesPow2, kKvBf16, SHORT><<<grid, 512, 0, s>>>(a);
  else prefill_kernel<DQK, DVO, kPagesAny, kKvBf16, SHORT><<<grid, 512, 0, s>>>(a);
}

template <int DQK, int DVO>
static void launch_prefill(const PrefillArgs& a, int pm, int kv, bool short_tiles, int grid, hipStream_t s) {
  if (short_tiles) launch_prefill<DQK, DVO, true>(a, pm, kv, grid, s);
  else launch_prefill<DQK, DVO, false>(a, pm, kv, grid, s);
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_paged_prefill(const pa_plan* plan, const void* q, const int32_t* qo_indptr,
                                      const pa_kv_cache* cache, const pa_page_table* table,
                                      const pa_attn_params* params, void* out, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  pa_status st = check_cache(cache, true);
  if (st != PA_OK) return st;
  int kv = cache->kv_dtype == PA_DTYPE_NVFP4        ? kKvFp4
           : cache->kv_dtype == PA_DTYPE_FP8_E4M3FN ? kKvFp8
                                                    : kKvBf16;
  if ((st = check_params(params, cache, kMaxPrefillGroup)) != PA_OK) return st;
  if ((st = check_plan_matches(plan, 2, params, cache, table, workspace_bytes)) != PA_OK) return st;
  if (plan->num_items == 0) return PA_OK;
  if (!q || !out || !qo_indptr) return fail(PA_ERR_INVALID_ARG, "q, qo_indptr or out is NULL");
  if (!workspace) return fail(PA_ERR_INVALID_ARG, "workspace is NULL");
  if (((uintptr_t)q | (uintptr_t)out | (uintptr_t)workspace) & 15)
    return fail(PA_ERR_UNSUPPORTED, "q, out and workspace must be 16-byte aligned");
  if ((uintptr_t)lse & 3) return fail(PA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  char* ws = (char*)workspace;
  PrefillArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const char*)cache->k;
  a.v = (const char*)cache->v;
  const int64_t unit = kv == kKvBf16 ? 2 : 1;  // bytes per stride unit
  a.k_sp = unit * cache->k_stride_page; a.k_sh = unit * cache->k_stride_head; a.k_st = unit * cache->k_stride_token;
  a.v_sp = unit * cache->v_stride_page; a.v_sh = unit * cache->v_stride_head; a.v_st = unit * cache->v_stride_token;
  a.k_sf = (const char*)cache->k_sf;
  a.v_sf = (const char*)cache->v_sf;
  a.ks_sp = cache->k_sf_stride_page; a.ks_sh = cache->k_sf_stride_head; a.ks_st = cache->k_sf_stride_token;
  a.vs_sp = cache->v_sf_stride_page; a.vs_sh = cache->v_sf_stride_head; a.vs_st = cache->v_sf_stride_token;
  a.v_scale = cache->v_scale;  // 1 for bf16 (checked)
  a.kv_indptr = table->kv_indptr;
  a.kv_indices = table->kv_indices;
  a.items = (const PrefillItem*)(ws + plan->items_offset);
  a.part_o = (float*)(ws + plan->partial_o_offset);
  a.part_lse = (float*)(ws + plan->partial_lse_offset);
  a.out = out;
  a.lse = lse;
  a.num_qo_heads = params->num_qo_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.group = params->num_qo_heads / cache->num_kv_heads;
  a.page_size = cache->page_size;
  a.page_shift = __builtin_ctz(cache->page_size);  // used only when page_size is a power of two
  a.window = params->window > 0 ? params->window : 0;
  a.causal = params->causal ? 1 : 0;
  a.out_fp32 = params->out_dtype == PA_DTYPE_FP32;
  // Scores are sm_scale * k_scale * q.k (k_scale is 1 for bf16).  The kernel takes |scale|
  // and transforms Q: sign bits flipped for a negative scale, zeroed for a zero one.
  const float sc = params->sm_scale * cache->k_scale;
  a.scale_log2 = (sc == 0.f ? 1.f : fabsf(sc)) * kLog2e;
  a.q_and = sc == 0.f ? 0u : 0xFFFFFFFFu;
  a.q_xor = sc < 0.f ? 0x80008000u : 0u;
  const int grid = plan->num_items * cache->num_kv_heads;
  hipStream_t s = (hipStream_t)stream;
  const int dqk = cache->head_dim_qk, dvo = cache->head_dim_vo;
  const int P = cache->page_size;
  if (plan->staged_pages > 0) {
    // Widen the table's NVFP4 pages into bf16 pages in the workspace, then run the bf16
    // kernel over them through an identity page list (k_scale is in scale_log2 and
    // v_scale in a.v_scale as before).
    const int64_t n = plan->staged_pages, H = cache->num_kv_heads;
    if (kv != kKvFp4 || plan->staged_offset < plan->partial_lse_offset ||
        plan->staged_offset + n * H * P * (dqk + dvo) * 2 + n * 4 > plan->workspace_bytes)
      return fail(PA_ERR_INVALID_ARG, "plan's widened-page region does not fit this cache");
    StageArgs g;
    g.k = a.k; g.v = a.v; g.k_sf = a.k_sf; g.v_sf = a.v_sf;
    g.k_sp = a.k_sp; g.k_sh = a.k_sh; g.k_st = a.k_st;
    g.v_sp = a.v_sp; g.v_sh = a.v_sh; g.v_st = a.v_st;
    g.ks_sp = a.ks_sp; g.ks_sh = a.ks_sh; g.ks_st = a.ks_st;
    g.vs_sp = a.vs_sp; g.vs_sh = a.vs_sh; g.vs_st = a.vs_st;
    g.kv_indices = a.kv_indices;
    g.k_out = (uint16_t*)(ws + plan->staged_offset);
    g.v_out = g.k_out + n * H * P * dqk;
    g.ident = (int32_t*)(g.v_out + n * H * P * dvo);
    g.num_kv_heads = (int32_t)H; g.page_size = P; g.dqk = dqk; g.dvo = dvo;
    nvfp4_stage_kernel<<<dim3((unsigned)n, (unsigned)H), 256, 0, s>>>(g);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_HIP, "nvfp4 widening launch: %s", hipGetErrorString(e));
    count_launches(1);
    kv = kKvBf16;
    a.k = (const char*)g.k_out;
    a.v = (const char*)g.v_out;
    a.k_sp = 2 * H * P * dqk; a.k_sh = 2 * (int64_t)P * dqk; a.k_st = 2 * dqk;
    a.v_sp = 2 * H * P * dvo; a.v_sh = 2 * (int64_t)P * dvo; a.v_st = 2 * dvo;
    a.k_sf = a.v_sf = nullptr;
    a.kv_indices = g.ident;
  }
  // The one-lookup-per-stage path forms byte offsets inside a page, and page strides, in
  // 32 bits.
  const bool page_fits_u32 = (int64_t)P * a.k_st + 2 * dqk < (int64_t(1) << 32) &&
                             (int64_t)P * a.v_st + 2 * dvo < (int64_t(1) << 32) &&
                             a.k_sp < (int64_t(1) << 32) && a.v_sp < (int64_t(1) << 32);
  const int pm = P % kKeyStage == 0 && page_fits_u32
                     ? kPagesStage
                     : ((P & (P - 1)) == 0 ? kPagesPow2 : kPagesAny);
  const bool short_tiles = plan->short_tiles != 0;
  // NVFP4 at 512/512 runs as two passes of the 512/256 kernel, one per half of the value
  // head_dim (the scores are computed in both): the 512/512 form's registers spill.  Each
  // pass reads its half of every V row and of its block scales, writes its half of each
  // output row, and has its own half of the partial-output workspace.
  const int parts = kv == kKvFp4 && dqk == 512 && dvo == 512 ? 2 : 1;
  const int pdvo = dvo / parts;
  const int64_t part_rows = (int64_t)plan->num_slots * cache->num_kv_heads * kPrefillTileRows;
  float* part_o0 = a.part_o;
  a.out_stride = dvo;
  for (int h = 0; h < parts; ++h) {
    if (h > 0) {
      a.v += pdvo / 2;        // packed E2M1: two elements a byte
      a.v_sf += pdvo / 16;    // one E4M3 scale per 16 elements
      a.out = (char*)a.out + (size_t)pdvo * (a.out_fp32 ? 4 : 2);
      a.part_o = part_o0 + part_rows * pdvo;
    }
    if (dqk == 512 && pdvo == 512) launch_prefill<512, 512>(a, pm, kv, short_tiles, grid, s);
    else if (dqk == 256) launch_prefill<256, 256>(a, pm, kv, short_tiles, grid, s);
    else launch_prefill<512, 256>(a, pm, kv, short_tiles, grid, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_HIP, "prefill kernel launch: %s", hipGetErrorString(e));
    count_launches(1);
    if (plan->num_merges > 0) {
      PrefillMergeArgs m;
      m.merges = (const PrefillMerge*)(ws + plan->merges_offset);
      m.part_o = a.part_o;
      m.part_lse = a.part_lse;
      m.out = a.out;
      m.out_stride = dvo;
      m.lse = a.lse;
      m.num_qo_heads = params->num_qo_heads;
      m.num_kv_heads = cache->num_kv_heads;
      m.group = a.group;
      m.out_fp32 = a.out_fp32;
      const dim3 mg(plan->num_merges, cache->num_kv_heads, kPrefillTileRows / 4);
      if (pdvo == 512) prefill_merge_kernel<512><<<mg, 256, 0, s>>>(m);
      else prefill_merge_kernel<256><<<mg, 256, 0, s>>>(m);
      e = hipGetLastError();
      if (e != hipSuccess) return fail(PA_ERR_HIP, "prefill merge launch: %s", hipGetErrorString(e));
      count_launches(1);
    }
  }
  return PA_OK;
}
