// Paged decode for gfx950: split-K partial kernel, log-sum-exp merge kernel, and the
// C entry points that plan-check and enqueue them.
//
// What is computed ("[None][feat] Run Gemma4 head_dim 512 attention on Triton",
// TensorRT-LLM pull request 17772, sections "Approach" and "Not covered"): for every
// request b and query head h, softmax(sm_scale * q . K^T) V over the request's visible
// keys, read through the page table from the combined HND cache, with the key axis cut
// into chunks whose partial results are merged by log-sum-exp weights (flash-decoding).
//
// Work decomposition.  The host planner flattens the (request, KV head, 16-token block)
// units and cuts them into equal pieces, one per wave (up to 2048 on the 256 CUs at two
// waves per SIMD), so every wave streams the same number of bytes and the whole grid is
// resident from start to end: no second round of workgroups, no tail of stragglers.  A
// piece is cut into segments at (request, KV head) boundaries; a segment's result goes to
// the output directly when it covers the whole pair, else to a workspace slot that the
// merge kernel combines.  The G query heads that share the KV head are computed together,
// so each K/V byte is read from HBM once for the whole group:
//   * S = K Q^T for a 16-key block is one 16x16 tile of v_mfma_f32_16x16x32_bf16 (keys
//     on M, the G heads padded to 16 on N, head_dim on K).  Each lane loads its K operand
//     straight from the page as 16-byte vectors (4 lanes cover 64 contiguous bytes of a key
//     row); Q sits in LDS with the same head_dim order.
//   * The online softmax keeps a running max and sum per head; the block max is a
//     cross-lane reduction over the 4 lanes that share a head.
//   * P V (bf16 and FP8 values) runs on the vector ALU one block behind S: each V load
//     instruction covers whole key rows (lane l holds 8 consecutive head_dim elements of
//     one row), each lane keeps G x 8 fp32 accumulators, and the block's probabilities
//     come from LDS as broadcast reads.  Block i's V rows are loaded while block i's
//     scores are computed and used in the next iteration; block i+1's keys are loaded
//     after block i's MFMAs.
//   * Waves never synchronise with each other; each one's results are deterministic.
// FP8 E4M3FN keys are widened to bf16 in registers (exact); k_scale is folded into the
// score scale and v_scale into the output.
// NVFP4 ("feat(attention): asymmetric VO-split NVFP4 paged prefill ...", FlashInfer pull
// request 3684, sections "Summary" and "NVFP4 split-KV correctness (added)"): each lane
// reads its keys' packed E2M1 bytes and their E4M3 block scales (one per 16 head_dim
// elements, from a tensor of their own addressed through the same page table), converts
// the nibbles and multiplies by the block scale.  Keys go through the fp16 MFMA: nibbles
// to fp16 pairs (v_cvt_scalef32_pk_f16_fp4 at scale 1) times the block scale in fp16
// (v_pk_mul_f16), exact since an E2M1 value times an E4M3 value has at most 6 significant
// bits and lies in [2^-10, 2688]; Q is staged in fp16, each segment's rows scaled by the
// power of two that brings their largest magnitude just below 2^15, so every bf16 query
// element converts exactly (short of 2^-29 of that largest one) and none overflows, and
// the factor comes back out of the score scale.  NVFP4 values go through the fp16 MFMA as
// well, still one block behind S: the contraction is taken over (half of head_dim, key), so
// each lane reads contiguous bytes of eight rows that share one scale block, and two rows'
// nibbles interleave into fp16 pairs of an A operand (no transpose); P, rounded to fp16,
// is the B operand.  The global k_scale / v_scale apply as for FP8.

#include <hip/hip_runtime.h>

#include <math.h>

#include <mutex>
#include <type_traits>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

struct DecodeArgs {
  const uint16_t* q;           // [B, Hq, DQK] bf16 bits
  const char* k;               // byte base of the K pool
  const char* v;               // byte base of the V pool
  int64_t k_sp, k_sh, k_st;    // element strides (NVFP4: bytes)
  int64_t v_sp, v_sh, v_st;
  const char* k_sf;            // NVFP4 block scales of K and V, else null
  const char* v_sf;
  int64_t ks_sp, ks_sh, ks_st; // block-scale strides, bytes
  int64_t vs_sp, vs_sh, vs_st;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const DecodeSegment* segs;   // head segment of wave w at index w, then further segments
  int32_t num_waves;
  int32_t park;                // the plan's deferred_partials
  int32_t group_last;          // the plan's grouped_partials
  void* out;                   // [B, Hq, DVO] fp32 or bf16
  float* lse;                  // [B, Hq] or null
  float* part_o;               // [slots, G, DVO] fp32
  float* part_lse;             // [slots, G], log2 domain
  int32_t num_qo_heads;
  int32_t group;
  int32_t page_size;
  int32_t out_fp32;
  float scale_log2;            // sm_scale * k_scale * log2(e)
  float v_scale;
};

// head_dim offset of the 8 bf16 operand elements that lane group g4 holds at MFMA step j.
// bf16 keys: one 16-byte load per step.  FP8 keys: one 16-byte load covers two steps.
// NVFP4 keys: lane group g4 holds the contiguous quarter [DQK/4 g4, DQK/4 (g4+1)) of the
// row (so its block scales are contiguous too); a 16-byte load covers four steps.
template <int KV, int DQK>
__device__ __forceinline__ int q_dim_of_step(int j, int g4) {
  if constexpr (KV == kKvBf16) return 32 * j + 8 * g4;
  else if constexpr (KV == kKvFp8) return 64 * (j >> 1) + 16 * g4 + 8 * (j & 1);
  else return (DQK / 4) * g4 + 8 * j;
}


// Eight waves per workgroup, one workgroup per CU: each wave runs its own piece (its
// segments one after the other) and never waits for the others.  They share LDS only to
// publish how many blocks each has done: a wave behind the CU's average raises its issue
// priority, because the hardware otherwise favours the older of the two waves on a SIMD,
// which then finishes far ahead of its partner and leaves the SIMD half-occupied for the
// rest of the kernel.
template <int DQK, int DVO, int KV, int GMAX>
__global__ __launch_bounds__(64 * kDecodeWavesPerGroup, 2) void decode_partial_kernel(DecodeArgs a) {
  constexpr int NWG = kDecodeWavesPerGroup;
  constexpr int UNIT = KV == kKvBf16 ? 2 : 1;    // bytes per stride unit
  constexpr int KROW = KV == kKvBf16 ? 2 * DQK : KV == kKvFp8 ? DQK : DQK / 2;  // K row bytes
  constexpr int VB8 = KV == kKvBf16 ? 16 : KV == kKvFp8 ? 8 : 4;  // bytes of 8 V elements
  constexpr int NSTEP = DQK / 32;                 // MFMA steps over head_dim
  constexpr int NKL = 16 * KROW / (64 * 16);      // 16-byte K loads per lane per block
  constexpr int NKSF = DQK / 64;                  // NVFP4: K block scales per lane (4 or 8)
  constexpr int LPR = DVO / 8;                    // lanes per V row (8 elements per lane)
  constexpr int RPI = 64 / LPR;                   // V rows per load instruction (1 or 2)
  constexpr int NVL = 16 / RPI;                   // V load instructions per block
  constexpr int QPITCH = DQK + 8;                 // LDS row pitch of Q (bf16), padded
  constexpr int QV = (GMAX * DQK / 8 + 63) / 64;  // 16-byte Q pieces per lane
  constexpr int TPD = DVO / 32;                   // NVFP4: P V MFMA tiles per block
  using vload_t = typename std::conditional<
      KV == kKvBf16, u32x4_t, typename std::conditional<KV == kKvFp8, u32x2_t, uint32_t>::type>::type;
  using ksf_t = typename std::conditional<NKSF == 8, u32x2_t, uint32_t>::type;
  using vq_t = typename std::conditional<TPD == 16, u32x2_t, uint32_t>::type;  // TPD nibbles
  // A split segment that is not the wave's last parks its result in LDS, and the wave writes
  // it to the workspace after its last segment: on this GPU a wave's loads and stores share
  // one in-order completion counter, so partial-result stores issued between segments made
  // the next segment's first loads wait for them under the full read load.  Parking needs
  // G x DVO floats per wave; where LDS is short, the P buffer keeps only the columns the
  // P V step reads, and instances that still do not fit store at once.  The same buffers
  // combine grouped last segments: consecutive waves of the workgroup whose last segments
  // belong to one split (request, KV head) each leave their result in LDS, and the last of
  // them to finish merges the group (in wave order) into one workspace slot.
  constexpr int PARK = GMAX * DVO + GMAX;         // floats: the outputs, then the log-sum-exps
  constexpr int PC = decode_p_columns(DQK, DVO, GMAX, KV == kKvFp4);  // P columns kept
  constexpr bool DEFER = decode_parks(DQK, DVO, GMAX, KV == kKvFp4);
  static_assert(QPITCH == DQK + 8, "the LDS budget assumes this Q pitch");

  __shared__ __attribute__((aligned(16))) uint16_t q_all[NWG][GMAX * QPITCH];
  __shared__ __attribute__((aligned(16))) float p_all[NWG][2][16][PC];  // P V runs one block behind
  __shared__ __attribute__((aligned(16))) float alpha_all[NWG][2][16];
  __shared__ __attribute__((aligned(16))) int progress[NWG];
  __shared__ __attribute__((aligned(16))) int grp_arrived[NWG];  // per group, at its first wave
  __shared__ __attribute__((aligned(16))) float park_all[DEFER ? NWG : 1][DEFER ? PARK : 4];
  // The planner decides from decode_lds_bytes whether split results can wait in LDS: it
  // must cover these buffers, and they must fit the CU.
  constexpr int kLdsUsed = sizeof(q_all) + sizeof(p_all) + sizeof(alpha_all) + sizeof(progress) +
                           sizeof(grp_arrived) + sizeof(park_all);
  static_assert(kLdsUsed <= decode_lds_bytes(DQK, DVO, GMAX, PC) || !DEFER, "LDS budget");
  static_assert(kLdsUsed <= kLdsBytesPerCu, "LDS of one CU");

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g4 = lane >> 4;
  const int n = lane & 15;
  const int G = a.group;
  const int qrow = n < G ? n : G - 1;  // MFMA columns past the group repeat the last head
  uint16_t* q_lds = q_all[wv];
  float (*p_lds)[16][PC] = p_all[wv];
  float* park = park_all[DEFER ? wv : 0];
  int parked_slot = -1;  // partial slot whose result waits in `park`
  // Writes the parked result to its workspace slot (the rows of heads 0 .. G-1 are
  // contiguous in both).
  auto flush_park = [&](int slot) {
    wave_lds_sync();
    float* dst = a.part_o + (int64_t)slot * G * DVO;
    for (int i = 4 * lane; i < G * DVO; i += 256) *(f32x4_t*)(dst + i) = *(const f32x4_t*)(park + i);
    if (lane < G) a.part_lse[(int64_t)slot * G + lane] = park[GMAX * DVO + lane];
  };
  // This wave's grouped result is in `park`: count it in, and if it is the group's last,
  // merge the members' results (waves first .. first + cnt - 1, in that order, whoever
  // finishes last) by the log-sum-exp rule into the group's slot.
  auto group_merge = [&](int slot, int cnt, int first) {
    wave_lds_sync();  // every lane's share of the result is in LDS before the count
    int before = 0;
    if (lane == 0)
      before = __hip_atomic_fetch_add(&grp_arrived[first], 1, __ATOMIC_ACQ_REL,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
    before = __builtin_amdgcn_readfirstlane(before);
    if (before != cnt - 1) return;
    wave_lds_sync();
    // Weights: lane 8 h + j takes member j's log-sum-exp of head h; the eight lanes of a
    // head reduce their max and sum, and each keeps its member's normalised weight.
    static_assert(GMAX * NWG <= 64, "one lane per (head, member)");
    const int wh = lane >> 3, wj = lane & 7;
    const bool wlive = wh < G && wj < cnt;
    const float l = wlive ? park_all[DEFER ? first + wj : 0][GMAX * DVO + wh] : -INFINITY;
    float mx = l;
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    mx = fmaxf(mx, __shfl_xor(mx, 4));
    float w = wlive ? exp2f(l - mx) : 0.f;
    float wsum = w;
    wsum += __shfl_xor(wsum, 1);
    wsum += __shfl_xor(wsum, 2);
    wsum += __shfl_xor(wsum, 4);
    if (wj == 0 && wh < G) a.part_lse[(int64_t)slot * G + wh] = mx + log2f(wsum);
    w = wlive ? w / wsum : 0.f;
    // Outputs: 256 floats per pass, all of one head (DVO is a multiple of 256); every
    // member's four floats are read before any is used, members past the group's size
    // repeating the last one with weight 0.
    float* dst = a.part_o + (int64_t)slot * G * DVO;
#pragma unroll
    for (int it = 0; it < GMAX * DVO / 256; ++it) {
      if (256 * it >= G * DVO) break;
      const int i = 256 * it + 4 * lane;
      const int h = 256 * it / DVO;
      f32x4_t v[NWG];
#pragma unroll
      for (int j = 0; j < NWG; ++j)
        v[j] = *(const f32x4_t*)(park_all[DEFER ? first + (j < cnt ? j : cnt - 1) : 0] + i);
      f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NWG; ++j) {
        const float wj_s = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), 8 * h + j));
        o[0] += wj_s * v[j][0];
        o[1] += wj_s * v[j][1];
        o[2] += wj_s * v[j][2];
        o[3] += wj_s * v[j][3];
      }
      *(f32x4_t*)(dst + i) = o;
    }
  };
  float (*alpha_lds)[16] = alpha_all[wv];
  const int wave = blockIdx.x * NWG + wv;
  // The wave's head segment names its further segments; each next record is requested when
  // the previous segment starts (a clamped index rather than a branch around the load).
  const bool active = wave < a.num_waves;
  const DecodeSegment head = a.segs[active ? wave : 0];
  const int n_seg = active ? 1 + (head.more_count & 0xFFFF) : 0;
  if (lane == 0) progress[wv] = 0;
  if constexpr (DEFER) {
    if (a.group_last) {  // uniform: every wave reaches this barrier
      if (lane == 0) grp_arrived[wv] = 0;
      lds_barrier();
    }
  }
  int done = 0;  // blocks this wave has finished

  u32x4_t kbuf[NKL];
  vload_t vbuf[NVL];
  ksf_t ksf;            // NVFP4: this lane's K block scales of the block (E4M3 codes)
  vq_t vq[8];           // NVFP4: TPD head_dim columns of eight V rows (see issue_v)
  uint32_t vsq[8];      // NVFP4: their block scales (E4M3 codes)
  float acc[GMAX][8];
  f32x4_t acc4[TPD];    // NVFP4: the P V tiles, one MFMA output each

  DecodeSegment sg_cur = head;
  for (int k = 0; k < n_seg; ++k) {
    const DecodeSegment sg = sg_cur;
    sg_cur = a.segs[k + 1 < n_seg ? head.more_begin + k : wave];
    const int t0 = sg.t_begin, t1 = sg.t_end;  // t1 > t0
    const int32_t* __restrict__ pages = a.kv_indices + sg.page_base;
    const int64_t k_head = (int64_t)sg.kvh * a.k_sh;
    const int64_t v_head = (int64_t)sg.kvh * a.v_sh;
    const int64_t ks_head = (int64_t)sg.kvh * a.ks_sh;
    const int64_t vs_head = (int64_t)sg.kvh * a.vs_sh;

    // Page and slot of key n of a block, clamped into the segment: every load is of a key
    // the segment owns, and clamped lanes are masked out of the softmax.  Block indices
    // past the end (the prefetch after the last block) land on the segment's last key.
    auto block_page = [&](int blk, int32_t& page, int32_t& slot) {
      int t = blk * 16 + n;
      t = t < t0 ? t0 : (t >= t1 ? t1 - 1 : t);
      token_page_slot(pages, t, a.page_size, page, slot);
    };
    auto issue_k = [&](int32_t page, int32_t slot) {
      const char* row = a.k + (row_elem_offset(page, 0, slot, a.k_sp, 0, a.k_st) + k_head) * UNIT;
      if constexpr (KV == kKvFp4) {
        const char* base = row + (KROW / 4) * g4;
#pragma unroll
        for (int l = 0; l < NKL; ++l) kbuf[l] = __builtin_nontemporal_load((const u32x4_t*)(base + 16 * l));
        const char* sf = a.k_sf + row_elem_offset(page, 0, slot, a.ks_sp, 0, a.ks_st) + ks_head + NKSF * g4;
        ksf = __builtin_nontemporal_load((const ksf_t*)sf);
      } else {
        const char* base = row + 16 * g4;
#pragma unroll
        for (int l = 0; l < NKL; ++l) kbuf[l] = __builtin_nontemporal_load((const u32x4_t*)(base + 64 * l));
      }
    };
    // Row byte offsets are formed on the vector ALU, lane n for key n of the block (all
    // sixteen at once), and each row's load takes its offset by v_readlane (or a lane
    // shuffle when two rows share an instruction): per-row 64-bit address arithmetic on the
    // scalar unit, which the CU's waves share, would serialise them.
    auto issue_v = [&](int32_t page, int32_t slot) {
      const int64_t voff = (row_elem_offset(page, 0, slot, a.v_sp, 0, a.v_st) + v_head) * UNIT;
      int64_t vsoff = 0;
      if constexpr (KV == kKvFp4) vsoff = row_elem_offset(page, 0, slot, a.vs_sp, 0, a.vs_st) + vs_head;
      if constexpr (KV == kKvFp4) {
        // NVFP4: lane (g4, n) reads keys 8 (g4 & 1) + r, r < 8, of the block, each at the TPD
        // contiguous columns DVO/2 (g4 >> 1) + TPD n, which lie in one 16-column scale block.
        const int kb = 8 * (g4 & 1);
        const char* vbase = a.v + ((DVO / 4) * (g4 >> 1) + (TPD / 2) * n);
        const char* sbase = a.v_sf + ((DVO / 2) * (g4 >> 1) + TPD * n) / 16;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int64_t off = shfl_i64(voff, kb + r);
          const int64_t soff = shfl_i64(vsoff, kb + r);
          vq[r] = __builtin_nontemporal_load((const vq_t*)(vbase + off));
          vsq[r] = __builtin_nontemporal_load((const uint8_t*)(sbase + soff));
        }
      } else {
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
          const int src = RPI * i + (RPI == 2 ? (lane >> 5) : 0);
          int64_t off;
          if constexpr (RPI == 1) off = readlane_i64(voff, src);  // src is wave-uniform
          else off = shfl_i64(voff, src);
          vbuf[i] = __builtin_nontemporal_load((const vload_t*)(a.v + off + (lane % LPR) * VB8));
        }
      }
    };
    // P V of one block: rescale the accumulators by the block's alpha, then add p * V with
    // the probabilities from LDS buffer `pb` and the V rows in vbuf.
    auto pv = [&](int pb) {
      if constexpr (KV == kKvFp4) {
        // NVFP4: O^T += V^T P^T on v_mfma_f32_16x16x32_f16, one MFMA per tile t < TPD.  The
        // 32-long contraction runs over (half x, key): A[i][(x, key)] = V[key][DVO/2 x + TPD i
        // + t] times the key's block scale (exact in fp16), B[(x, key)][(x', h)] = P[key][h]
        // when x = x', else 0.  Output column (x', h) of tile t is head h at head_dim columns
        // DVO/2 x' + TPD i + t, so lane (g4, n) ends with head n & 7 at the 4 TPD columns
        // from DVO/2 (n >> 3) + 4 TPD g4 (acc4[t][r] at column TPD r + t).
        // Rescale only when some head's running max moved (a wave-uniform branch with no
        // load inside): after a segment's first blocks the max rarely changes.
        const float al = alpha_lds[pb][n & 7];
        if (__builtin_amdgcn_ballot_w64(al != 1.f)) {
#pragma unroll
          for (int t = 0; t < TPD; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc4[t][r] *= al;
        }
        const bool on = (g4 >> 1) == (n >> 3);
        const int kb = 8 * (g4 & 1);
        u32x4_t pw;
#pragma unroll
        for (int c = 0; c < 4; ++c)
          pw[c] = on ? pack_f16(p_lds[pb][kb + 2 * c][n & 7], p_lds[pb][kb + 2 * c + 1][n & 7]) : 0u;
        const f16x8_t bop = __builtin_bit_cast(f16x8_t, pw);
        f16x2_t sc2[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          sc2[c] = f16x2_t{(_Float16)fp8_to_f32<0>(vsq[2 * c]), (_Float16)fp8_to_f32<0>(vsq[2 * c + 1])};
#pragma unroll
        for (int w = 0; w < TPD / 8; ++w) {
          f16x2_t col[4][8];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if constexpr (TPD == 16) fp4x8_pair_to_f16x2(vq[2 * c][w], vq[2 * c + 1][w], col[c]);
            else fp4x8_pair_to_f16x2(vq[2 * c], vq[2 * c + 1], col[c]);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const f16x2_t x0 = col[0][e] * sc2[0], x1 = col[1][e] * sc2[1];
            const f16x2_t x2 = col[2][e] * sc2[2], x3 = col[3][e] * sc2[3];
            const f16x8_t aop = {x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
            acc4[8 * w + e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop, bop, acc4[8 * w + e], 0, 0, 0);
          }
        }
      } else {
      {
        float al[GMAX];
#pragma unroll
        for (int h = 0; h < GMAX; ++h) al[h] = alpha_lds[pb][h];
#pragma unroll
        for (int h = 0; h < GMAX; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] *= al[h];
      }
#pragma unroll
      for (int i = 0; i < NVL; ++i) {
        const int tk = RPI * i + (RPI == 2 ? (lane >> 5) : 0);
        float p[GMAX];
#pragma unroll
        for (int h = 0; h < GMAX; ++h) p[h] = p_lds[pb][tk][h];
        float vf[8];
        if constexpr (KV == kKvBf16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vf[2 * e] = bf16_lo(vbuf[i][e]);
            vf[2 * e + 1] = bf16_hi(vbuf[i][e]);
          }
        } else {
          fp8x4_to_f32(vbuf[i][0], vf);
          fp8x4_to_f32(vbuf[i][1], vf + 4);
        }
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
          if (GMAX == 1 || h < G) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p[h], vf[e], acc[h][e]);
          }
        }
      }
      }
    };

    // ---- Q rows of the group, the first block's page lookup and its keys, all in flight
    // together (the Q loads go first; their LDS store waits only for them).  No load
    // below sits behind a branch: a load on one side of a branch makes the compiler wait
    // for every outstanding load where the paths join, which would serialise the pipeline.
    const uint16_t* qsrc = a.q + ((int64_t)sg.b * a.num_qo_heads + (int64_t)sg.kvh * G) * DQK;
    u32x4_t qv_pre[QV];
#pragma unroll
    for (int r = 0; r < QV; ++r) {
      const int idx = lane + 64 * r;
      const int row = idx / (DQK / 8), c8 = idx % (DQK / 8);
      qv_pre[r] = *(const u32x4_t*)(qsrc + (row < G ? row : G - 1) * DQK + c8 * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
    int blk = t0 / 16;
    const int blk_end = (t1 + 15) / 16;
    int32_t page_c, slot_c;
    block_page(blk, page_c, slot_c);
    issue_k(page_c, slot_c);
    float seg_scale = a.scale_log2;  // log2-domain factor of the raw scores
    if constexpr (KV == kKvFp4) {
      // Q to fp16, scaled by 2^sh so that max |q| lies in [2^14, 2^15).
      float qm = 0.f;
#pragma unroll
      for (int r = 0; r < QV; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          qm = fmaxf(qm, fmaxf(fabsf(bf16_lo(qv_pre[r][e])), fabsf(bf16_hi(qv_pre[r][e]))));
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) qm = fmaxf(qm, shfl_xor_f(qm, o));
      int ex = 0;
      frexpf(qm, &ex);  // qm < 2^ex
      const int sh = qm > 0.f ? min(max(15 - ex, -126), 126) : 0;
      const float up = __builtin_ldexpf(1.f, sh);
      seg_scale = a.scale_log2 * __builtin_ldexpf(1.f, -sh);
#pragma unroll
      for (int r = 0; r < QV; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          qv_pre[r][e] = pack_f16(bf16_lo(qv_pre[r][e]) * up, bf16_hi(qv_pre[r][e]) * up);
    }
#pragma unroll
    for (int r = 0; r < QV; ++r) {
      const int idx = lane + 64 * r;
      const int row = idx / (DQK / 8), c8 = idx % (DQK / 8);
      if (row < G) *(u32x4_t*)(q_lds + row * QPITCH + c8 * 8) = qv_pre[r];
    }
    wave_lds_sync();

    float m_run = -INFINITY;  // per head n, log2 domain
    float l_run = 0.f;        // this lane's share of the sum for head n
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
    for (int t = 0; t < TPD; ++t) acc4[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    int iter = 0;
    for (; blk < blk_end; ++blk, ++iter) {
      const int cur = iter & 1;
      // ---- page index of the next block, which this iteration's key prefetch needs.
      int32_t page_n, slot_n;
      block_page(blk + 1, page_n, slot_n);
      // ---- P V of the previous block, then this block's V rows (used next iteration).
      if (iter > 0) {
        pv(cur ^ 1);
        wave_lds_sync();
      }
      issue_v(page_c, slot_c);
      // ---- S^T = K Q^T for the 16 keys of this block (keys on rows, heads on columns).
      f32x4_t s = {0.f, 0.f, 0.f, 0.f};
      float kbs[NKSF];  // NVFP4: the lane's K block scales as fp32
      if constexpr (KV == kKvFp4) {
        if constexpr (NKSF == 8) {
          fp8x4_to_f32(ksf[0], kbs);
          fp8x4_to_f32(ksf[1], kbs + 4);
        } else {
          fp8x4_to_f32(ksf, kbs);
        }
      }
#pragma unroll
      for (int j = 0; j < NSTEP; ++j) {
        if constexpr (KV == kKvFp4) {
          const f16x8_t kf = fp4x8_to_f16_scaled(kbuf[j >> 2][j & 3], (_Float16)kbs[j >> 1]);
          const u32x4_t qv = *(const u32x4_t*)(q_lds + qrow * QPITCH + q_dim_of_step<KV, DQK>(j, g4));
          s = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, __builtin_bit_cast(f16x8_t, qv), s, 0, 0, 0);
          continue;
        }
        bf16x8_t kf;
        if constexpr (KV == kKvBf16) {
          kf = __builtin_bit_cast(bf16x8_t, kbuf[j]);
        } else {
          const u32x4_t raw = kbuf[j >> 1];
          const u32x2_t lo = fp8x4_to_bf16x4(raw[(j & 1) * 2 + 0]);
          const u32x2_t hi = fp8x4_to_bf16x4(raw[(j & 1) * 2 + 1]);
          const u32x4_t packed = {lo[0], lo[1], hi[0], hi[1]};
          kf = __builtin_bit_cast(bf16x8_t, packed);
        }
        const u32x4_t qv = *(const u32x4_t*)(q_lds + qrow * QPITCH + q_dim_of_step<KV, DQK>(j, g4));
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, __builtin_bit_cast(bf16x8_t, qv), s, 0, 0, 0);
      }
      // ---- prefetch the next block's keys.
      issue_k(page_n, slot_n);

      // ---- online softmax over the block; lane (g4, n) holds keys 4*g4 + i of head n.
      float sc[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = blk * 16 + 4 * g4 + i;
        sc[i] = (t >= t0 && t < t1) ? s[i] * seg_scale : -INFINITY;
        mx = fmaxf(mx, sc[i]);
      }
      mx = max_xor16(mx);
      mx = max_xor32(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);  // every block holds a visible key
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(sc[i] - m_new);
        psum += p;
        if (n < PC) p_lds[cur][4 * g4 + i][n] = p;
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (g4 == 0) alpha_lds[cur][n] = alpha;
      wave_lds_sync();
      page_c = page_n;
      slot_c = slot_n;
      // ---- issue priority from the workgroup's progress (plain LDS words; a stale value
      // only delays the adjustment by an iteration): highest while behind the CU's
      // average, low within a block ahead of it, lowest further ahead.
      ++done;
      if (lane == 0) progress[wv] = done;
      int sum = 0;
#pragma unroll
      for (int x = 0; x < NWG; ++x) sum += progress[x];
      const int lag = sum - done * NWG;  // NWG x (blocks behind the CU's average)
      if (lag > 0) __builtin_amdgcn_s_setprio(3);
      else if (lag > -NWG) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
    pv((iter - 1) & 1);

    // ---- segment result: the sum over the 4 lanes of a head, and (two rows per V load)
    // the accumulator halves.  Lane h < 16 then holds head h's max and sum.
    l_run = sum_xor32(sum_xor16(l_run));
    if constexpr (RPI == 2 && KV != kKvFp4) {
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] += shfl_xor_f(acc[h][e], 32);
    }
    const int h0 = sg.kvh * G;
    // The last segment carries its group: bits 16-23 of more_count its size (0: none),
    // bits 24-31 its first wave within the workgroup.
    const int grp_n = (sg.more_count >> 16) & 0xFF;
    const bool to_group = DEFER && k + 1 == n_seg && grp_n >= 2;
    if constexpr (DEFER) {
      if (to_group && parked_slot >= 0) {  // the buffer takes this result: write out the last
        flush_park(parked_slot);
        parked_slot = -1;
      }
    }
    const bool to_park =
        DEFER && sg.slot >= 0 && (to_group || (a.park && k + 1 < n_seg && parked_slot < 0));
    if constexpr (KV == kKvFp4) {
      // Lane (g4, n): head n & 7 at the 4 TPD columns from DVO/2 (n >> 3) + 4 TPD g4.
      const int h = n & 7;
      const float lh = __builtin_bit_cast(
          float, __builtin_amdgcn_ds_bpermute(h << 2, __builtin_bit_cast(int, l_run)));
      if (h < G) {
        const float inv = lh > 0.f ? a.v_scale / lh : 0.f;
        const int d0 = (DVO / 2) * (n >> 3) + 4 * TPD * g4;
        float o[4 * TPD];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int t = 0; t < TPD; ++t) o[TPD * r + t] = acc4[t][r] * inv;
        if (to_park) {
#pragma unroll
          for (int c = 0; c < TPD; ++c)
            *(f32x4_t*)(park + h * DVO + d0 + 4 * c) = f32x4_t{o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]};
        } else if (sg.slot >= 0) {
          float* dst = a.part_o + ((int64_t)sg.slot * G + h) * DVO + d0;
#pragma unroll
          for (int c = 0; c < TPD; ++c)
            *(f32x4_t*)(dst + 4 * c) = f32x4_t{o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]};
        } else {
          const int64_t off = ((int64_t)sg.b * a.num_qo_heads + h0 + h) * DVO + d0;
          if (a.out_fp32) {
            float* dst = (float*)a.out + off;
#pragma unroll
            for (int c = 0; c < TPD; ++c)
              *(f32x4_t*)(dst + 4 * c) = f32x4_t{o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]};
          } else {
#pragma unroll
            for (int c = 0; c < TPD / 2; ++c) {
              const u32x4_t pk = {pack_bf16(o[8 * c], o[8 * c + 1]), pack_bf16(o[8 * c + 2], o[8 * c + 3]),
                                  pack_bf16(o[8 * c + 4], o[8 * c + 5]), pack_bf16(o[8 * c + 6], o[8 * c + 7])};
              *(u32x4_t*)((uint16_t*)a.out + off + 8 * c) = pk;
            }
          }
        }
      }
    } else if (lane < LPR) {
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        if (h >= G) continue;
        const float lh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_run), h));
        const float inv = lh > 0.f ? a.v_scale / lh : 0.f;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = acc[h][e] * inv;
        if (to_park) {
          float* dst = park + h * DVO + lane * 8;
          *(f32x4_t*)dst = f32x4_t{o[0], o[1], o[2], o[3]};
          *(f32x4_t*)(dst + 4) = f32x4_t{o[4], o[5], o[6], o[7]};
        } else if (sg.slot >= 0) {
          float* dst = a.part_o + ((int64_t)sg.slot * G + h) * DVO + lane * 8;
          *(f32x4_t*)dst = f32x4_t{o[0], o[1], o[2], o[3]};
          *(f32x4_t*)(dst + 4) = f32x4_t{o[4], o[5], o[6], o[7]};
        } else {
          const int64_t off = ((int64_t)sg.b * a.num_qo_heads + h0 + h) * DVO + lane * 8;
          if (a.out_fp32) {
            float* dst = (float*)a.out + off;
            *(f32x4_t*)dst = f32x4_t{o[0], o[1], o[2], o[3]};
            *(f32x4_t*)(dst + 4) = f32x4_t{o[4], o[5], o[6], o[7]};
          } else {
            u32x4_t pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) pk[e] = pack_bf16(o[2 * e], o[2 * e + 1]);
            *(u32x4_t*)((uint16_t*)a.out + off) = pk;
          }
        }
      }
    }
    if (lane < G) {
      const float lg = m_run + log2f(l_run);  // log2 domain; l_run > 0 here
      if (to_park) park[GMAX * DVO + lane] = lg;
      else if (sg.slot >= 0) a.part_lse[(int64_t)sg.slot * G + lane] = lg;
      else if (a.lse) a.lse[(int64_t)sg.b * a.num_qo_heads + h0 + lane] = lg * kLn2;
    }
    if (to_group) {
      if constexpr (DEFER) group_merge(sg.slot, grp_n, (uint32_t)sg.more_count >> 24);
    } else if (to_park) {
      parked_slot = sg.slot;
    }
  }
  if constexpr (DEFER) {
    if (parked_slot >= 0) flush_park(parked_slot);
  }
}

struct MergeArgs {
  const MergeItem* merges;
  const float* part_o;     // [slots, G, DVO]
  const float* part_lse;   // [slots, G], log2 domain
  void* out;
  float* lse;
  int32_t num_qo_heads;
  int32_t group;
  int32_t out_fp32;
};

// One wave per (merged (request, KV head), head of the group): log-sum-exp weights over
// the segments, then the weighted sum of the segment outputs in segment order.  The rows
// do not depend on the weights, so the log-sum-exps of up to 64 segments (one per lane) and
// the rows of the first 16 segments are requested together before any of them is used: a
// pair of up to 16 segments costs one memory round trip.  Further rows are read 8 at a
// time.  A pair with no segments (no keys) gets a zero output and lse -inf.
template <int DVO>
__global__ __launch_bounds__(64) void decode_merge_kernel(MergeArgs a) {
  constexpr int EPT = DVO / 64;
  constexpr int UN0 = 16;  // rows requested with the log-sum-exps
  constexpr int UN = 8;    // rows in flight per later step
  const MergeItem mi = a.merges[blockIdx.x];
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int G = a.group;
  const int n = mi.num_slots;
  float o[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) o[e] = 0.f;
  float mx = -INFINITY, wsum = 0.f;
  if (n > 0) {
    const float* lse_col = a.part_lse + (int64_t)mi.slot_begin * G + h;
    const int64_t rstride = (int64_t)G * DVO;
    const float* src0 = a.part_o + ((int64_t)mi.slot_begin * G + h) * DVO + lane * EPT;
    // Lane c: log-sum-exp of segment min(c, n - 1); rows 0 .. UN0 - 1, clamped to the last
    // segment (the clamped copies get weight 0).
    const float lv0 = lse_col[(int64_t)min(lane, n - 1) * G];
    f32x4_t x0[UN0][EPT / 4];
#pragma unroll
    for (int u = 0; u < UN0; ++u)
#pragma unroll
      for (int e = 0; e < EPT / 4; ++e)
        x0[u][e] = *(const f32x4_t*)(src0 + (int64_t)min(u, n - 1) * rstride + 4 * e);
    mx = lane < n ? lv0 : -INFINITY;
    for (int c = 64 + lane; c < n; c += 64) mx = fmaxf(mx, lse_col[(int64_t)c * G]);
    mx = max_xor16(max_xor32(mx));
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, m));
    const float mu = mx == -INFINITY ? 0.f : mx;
    float w = lane < n ? exp2f(lv0 - mu) : 0.f;
    float wpart = w;
#pragma unroll
    for (int u = 0; u < UN0; ++u) {
      const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
#pragma unroll
      for (int e = 0; e < EPT / 4; ++e)
#pragma unroll
        for (int v = 0; v < 4; ++v) o[4 * e + v] = fmaf(wu, x0[u][e][v], o[4 * e + v]);
    }
    // The rest, in segment order: rows UN0 .. of the first 64, then 64 at a time (their
    // log-sum-exps one per lane again).
    int c = UN0;
    for (int c0 = 0; c0 < n; c0 += 64) {
      const int cn = min(64, n - c0);
      if (c0 > 0) {
        const float lv = lse_col[(int64_t)(c0 + min(lane, cn - 1)) * G];
        w = lane < cn ? exp2f(lv - mu) : 0.f;
        wpart += w;
        c = 0;
      }
      const float* src = src0 + (int64_t)c0 * rstride;
      for (; c + UN <= cn; c += UN) {
        f32x4_t x[UN][EPT / 4];
#pragma unroll
        for (int u = 0; u < UN; ++u)
#pragma unroll
          for (int e = 0; e < EPT / 4; ++e) x[u][e] = *(const f32x4_t*)(src + (c + u) * rstride + 4 * e);
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), c + u));
#pragma unroll
          for (int e = 0; e < EPT / 4; ++e)
#pragma unroll
            for (int v = 0; v < 4; ++v) o[4 * e + v] = fmaf(wu, x[u][e][v], o[4 * e + v]);
        }
      }
      for (; c < cn; ++c) {
        const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), c));
#pragma unroll
        for (int e = 0; e < EPT / 4; ++e) {
          const f32x4_t x = *(const f32x4_t*)(src + c * rstride + 4 * e);
#pragma unroll
          for (int v = 0; v < 4; ++v) o[4 * e + v] = fmaf(wu, x[v], o[4 * e + v]);
        }
      }
    }
    wsum = sum_xor16(sum_xor32(wpart));
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) wsum += shfl_xor_f(wsum, m);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int hq = a.num_qo_heads;
  const int64_t off = ((int64_t)mi.b * hq + mi.kvh * G + h) * DVO + lane * EPT;
  if (a.out_fp32) {
    float* dst = (float*)a.out + off;
#pragma unroll
    for (int e = 0; e < EPT; e += 4)
      *(f32x4_t*)(dst + e) = f32x4_t{o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv};
  } else {
    uint32_t* dst = (uint32_t*)((uint16_t*)a.out + off);
#pragma unroll
    for (int e = 0; e < EPT; e += 2) dst[e / 2] = pack_bf16(o[e] * inv, o[e + 1] * inv);
  }
  if (a.lse && lane == 0)
    a.lse[(int64_t)mi.b * hq + mi.kvh * G + h] = wsum > 0.f ? (mx + log2f(wsum)) * kLn2 : -INFINITY;
}

// Copies the rows of one (request, KV head) in logical order, through the same address
// path as the attention kernels.  One workgroup per key.  NVFP4: each output row is the
// packed data row followed by its block-scale row.
struct GatherArgs {
  const char* k;
  const char* v;
  int64_t k_sp, k_sh, k_st, v_sp, v_sh, v_st;        // strides in stored units
  const char* k_sf;                                   // NVFP4 block scales, else null
  const char* v_sf;
  int64_t ks_sp, ks_sh, ks_st, vs_sp, vs_sh, vs_st;  // bytes
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  int32_t b, head, page_size, esz;                    // esz: bytes per stride unit
  int32_t k_row_bytes, v_row_bytes;                   // data bytes per row
  int32_t ks_row_bytes, vs_row_bytes;                 // block-scale bytes per row (0: none)
  char* k_out;
  char* v_out;
};

__device__ __forceinline__ void copy_row16(char* dst, const char* src, int bytes) {
  for (int c = threadIdx.x; c < bytes / 16; c += 64)
    *(u32x4_t*)(dst + 16 * c) = *(const u32x4_t*)(src + 16 * c);
}

__global__ __launch_bounds__(64) void gather_kv_kernel(GatherArgs a) {
  const int t = blockIdx.x;
  int32_t page, slot;
  token_page_slot(a.kv_indices + a.kv_indptr[a.b], t, a.page_size, page, slot);
  const int64_t k_out_row = a.k_row_bytes + a.ks_row_bytes, v_out_row = a.v_row_bytes + a.vs_row_bytes;
  char* ko = a.k_out + (int64_t)t * k_out_row;
  char* vo = a.v_out + (int64_t)t * v_out_row;
  copy_row16(ko, a.k + row_elem_offset(page, a.head, slot, a.k_sp, a.k_sh, a.k_st) * a.esz, a.k_row_bytes);
  copy_row16(vo, a.v + row_elem_offset(page, a.head, slot, a.v_sp, a.v_sh, a.v_st) * a.esz, a.v_row_bytes);
  if (a.ks_row_bytes > 0) {
    copy_row16(ko + a.k_row_bytes,
               a.k_sf + row_elem_offset(page, a.head, slot, a.ks_sp, a.ks_sh, a.ks_st), a.ks_row_bytes);
    copy_row16(vo + a.v_row_bytes,
               a.v_sf + row_elem_offset(page, a.head, slot, a.vs_sp, a.vs_sh, a.vs_st), a.vs_row_bytes);
  }
}

__global__ void fp8_to_f32_kernel(const uint8_t* codes, float* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (4 * i >= n) return;
  uint32_t w = 0;
  for (int u = 0; u < 4 && 4 * i + u < n; ++u) w |= (uint32_t)codes[4 * i + u] << (8 * u);
  float f[4];
  fp8x4_to_f32(w, f);
  for (int u = 0; u < 4 && 4 * i + u < n; ++u) out[4 * i + u] = f[u];
}

template <int DQK, int DVO, int KV>
static hipError_t launch_decode_dims(const DecodeArgs& a, int gmax, int grid, hipStream_t s) {
  switch (gmax) {
    case 1: decode_partial_kernel<DQK, DVO, KV, 1><<<grid, 64 * kDecodeWavesPerGroup, 0, s>>>(a); break;
    case 2: decode_partial_kernel<DQK, DVO, KV, 2><<<grid, 64 * kDecodeWavesPerGroup, 0, s>>>(a); break;
    case 3: decode_partial_kernel<DQK, DVO, KV, 3><<<grid, 64 * kDecodeWavesPerGroup, 0, s>>>(a); break;
    case 4: decode_partial_kernel<DQK, DVO, KV, 4><<<grid, 64 * kDecodeWavesPerGroup, 0, s>>>(a); break;
    case 6: decode_partial_kernel<DQK, DVO, KV, 6><<<grid, 64 * kDecodeWavesPerGroup, 0, s>>>(a); break;
    default: decode_partial_kernel<DQK, DVO, KV, 8><<<grid, 64 * kDecodeWavesPerGroup, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

template <int KV>
static hipError_t launch_decode_kv(const DecodeArgs& a, int dqk, int dvo, int gmax, int grid,
                                   hipStream_t s) {
  if (dqk == 512 && dvo == 512) return launch_decode_dims<512, 512, KV>(a, gmax, grid, s);
  if (dqk == 256 && dvo == 256) return launch_decode_dims<256, 256, KV>(a, gmax, grid, s);
  return launch_decode_dims<512, 256, KV>(a, gmax, grid, s);
}

static hipError_t launch_decode(const DecodeArgs& a, int dqk, int dvo, int kv_dtype, int gmax,
                                int grid, hipStream_t s) {
  if (kv_dtype == PA_DTYPE_BF16) return launch_decode_kv<kKvBf16>(a, dqk, dvo, gmax, grid, s);
  if (kv_dtype == PA_DTYPE_FP8_E4M3FN) return launch_decode_kv<kKvFp8>(a, dqk, dvo, gmax, grid, s);
  return launch_decode_kv<kKvFp4>(a, dqk, dvo, gmax, grid, s);
}

// ---- Workspace for callers that cannot allocate (pa_paged_decode_static).
// A file-scope device array stands in for the caller's workspace: the uploaded plan and the
// split partials.  Each GPU the library runs on holds its own copy, zeroed when the code
// object is loaded and kept until the process ends.  In host code `scratch` is only a
// stand-in for the symbol; its device address comes from hipGetSymbolAddress, once per
// device with that device current, and only that address is passed to kernels.
constexpr size_t kStaticWorkspaceBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static pa_status static_workspace(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "device %d: the static workspace serves devices 0..%d", dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" {


pa_status pa_plan_upload(const pa_plan* plan, const void* plan_buf_host, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!plan || !plan_buf_host) return fail(PA_ERR_INVALID_ARG, "plan or plan buffer is NULL");
  if (plan->plan_bytes == 0) return PA_OK;
  if (!workspace) return fail(PA_ERR_INVALID_ARG, "workspace is NULL");
  if ((int64_t)workspace_bytes < plan->workspace_bytes)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, plan needs %lld",
                workspace_bytes, (long long)plan->workspace_bytes);
  hipError_t e = hipMemcpyAsync(workspace, plan_buf_host, (size_t)plan->plan_bytes,
                                hipMemcpyHostToDevice, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  return PA_OK;
}

// Argument checks of a decode run; *nothing_to_do is set when the plan holds no work.
static pa_status decode_check(const pa_plan* plan, const void* q, const pa_kv_cache* cache,
                              const pa_page_table* table, const pa_attn_params* params,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              bool* nothing_to_do) {
  *nothing_to_do = false;
  pa_status st = check_cache(cache, true);
  if (st != PA_OK) return st;
  if ((st = check_params(params, cache, kMaxDecodeGroup)) != PA_OK) return st;
  if ((st = check_plan_matches(plan, 1, params, cache, table, workspace_bytes)) != PA_OK) return st;
  if (plan->num_items == 0 && plan->num_merges == 0) {
    *nothing_to_do = true;
    return PA_OK;
  }
  if (!q || !out) return fail(PA_ERR_INVALID_ARG, "q or out is NULL");
  if (!workspace) return fail(PA_ERR_INVALID_ARG, "workspace is NULL");
  if (((uintptr_t)q | (uintptr_t)out | (uintptr_t)workspace) & 15)
    return fail(PA_ERR_UNSUPPORTED, "q, out and workspace must be 16-byte aligned");
  if ((uintptr_t)lse & 3) return fail(PA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  return PA_OK;
}

static pa_status decode_enqueue(const pa_plan* plan, const void* q, const pa_kv_cache* cache,
                                const pa_page_table* table, const pa_attn_params* params,
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream, bool run_partial, bool run_merge) {
  bool nothing = false;
  pa_status st = decode_check(plan, q, cache, table, params, out, lse, workspace,
                              workspace_bytes, &nothing);
  if (st != PA_OK || nothing) return st;

  const int group = params->num_qo_heads / cache->num_kv_heads;
  const int gmax = decode_gmax(group);
  char* ws = (char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const bool out_fp32 = params->out_dtype == PA_DTYPE_FP32;
  float* part_o = (float*)(ws + plan->partial_o_offset);
  float* part_lse = (float*)(ws + plan->partial_lse_offset);
  if (run_partial && plan->num_workers > 0) {
    DecodeArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const char*)cache->k;
    a.v = (const char*)cache->v;
    a.k_sp = cache->k_stride_page; a.k_sh = cache->k_stride_head; a.k_st = cache->k_stride_token;
    a.v_sp = cache->v_stride_page; a.v_sh = cache->v_stride_head; a.v_st = cache->v_stride_token;
    a.k_sf = (const char*)cache->k_sf;
    a.v_sf = (const char*)cache->v_sf;
    a.ks_sp = cache->k_sf_stride_page; a.ks_sh = cache->k_sf_stride_head; a.ks_st = cache->k_sf_stride_token;
    a.vs_sp = cache->v_sf_stride_page; a.vs_sh = cache->v_sf_stride_head; a.vs_st = cache->v_sf_stride_token;
    a.kv_indptr = table->kv_indptr;
    a.kv_indices = table->kv_indices;
    a.segs = (const DecodeSegment*)(ws + plan->items_offset);
    a.num_waves = plan->num_workers;
    a.park = plan->deferred_partials;
    a.group_last = plan->grouped_partials;
    a.out = out;
    a.lse = lse;
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.num_qo_heads = params->num_qo_heads;
    a.group = group;
    a.page_size = cache->page_size;
    a.out_fp32 = out_fp32;
    a.scale_log2 = params->sm_scale * cache->k_scale * kLog2e;
    a.v_scale = cache->v_scale;
    const int grid = (plan->num_workers + kDecodeWavesPerGroup - 1) / kDecodeWavesPerGroup;
    hipError_t e = launch_decode(a, cache->head_dim_qk, cache->head_dim_vo, cache->kv_dtype, gmax,
                                 grid, s);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "decode kernel launch: %s", hipGetErrorString(e));
    count_launches(1);
  }
  if (run_merge && plan->num_merges > 0) {
    MergeArgs m;
    m.merges = (const MergeItem*)(ws + plan->merges_offset);
    m.part_o = part_o;
    m.part_lse = part_lse;
    m.out = out;
    m.lse = lse;
    m.num_qo_heads = params->num_qo_heads;
    m.group = group;
    m.out_fp32 = out_fp32;
    dim3 mg(plan->num_merges, group);
    if (cache->head_dim_vo == 512) decode_merge_kernel<512><<<mg, 64, 0, s>>>(m);
    else decode_merge_kernel<256><<<mg, 64, 0, s>>>(m);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_HIP, "merge kernel launch: %s", hipGetErrorString(e));
    count_launches(1);
  }
  return PA_OK;
}

pa_status pa_paged_decode(const pa_plan* plan, const void* q, const pa_kv_cache* cache,
                          const pa_page_table* table, const pa_attn_params* params,
                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return decode_enqueue(plan, q, cache, table, params, out, lse, workspace, workspace_bytes,
                        stream, true, true);
}

pa_status pa_paged_decode_partial(const pa_plan* plan, const void* q, const pa_kv_cache* cache,
                                  const pa_page_table* table, const pa_attn_params* params,
                                  void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return decode_enqueue(plan, q, cache, table, params, out, lse, workspace, workspace_bytes,
                        stream, true, false);
}

pa_status pa_paged_decode_merge(const pa_plan* plan, const void* q, const pa_kv_cache* cache,
                                const pa_page_table* table, const pa_attn_params* params,
                                void* out, float* lse, void* workspace, size_t workspace_bytes,
                                void* stream) {
  return decode_enqueue(plan, q, cache, table, params, out, lse, workspace, workspace_bytes,
                        stream, false, true);
}

pa_status pa_paged_decode_static(const pa_plan* plan, const void* plan_buf_host, const void* q,
                                 const pa_kv_cache* cache, const pa_page_table* table,
                                 const pa_attn_params* params, void* out, float* lse,
                                 void* stream) {
  if (!plan || !plan_buf_host) return fail(PA_ERR_INVALID_ARG, "plan or plan buffer is NULL");
  if (plan->workspace_bytes < 0 || (uint64_t)plan->workspace_bytes > kStaticWorkspaceBytes)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL,
                "the plan needs a %lld-byte workspace; the static workspace holds %zu bytes "
                "(use pa_paged_decode with a workspace of your own)",
                (long long)plan->workspace_bytes, kStaticWorkspaceBytes);
  void* ws = nullptr;
  pa_status st = static_workspace(&ws);
  if (st != PA_OK) return st;
  bool nothing = false;
  st = decode_check(plan, q, cache, table, params, out, lse, ws, kStaticWorkspaceBytes, &nothing);
  if (st != PA_OK || nothing) return st;
  // The plan goes into the workspace first, in stream order (no allocation).
  if (plan->plan_bytes > 0) {
    hipError_t e = hipMemcpyAsync(ws, plan_buf_host, (size_t)plan->plan_bytes,
                                  hipMemcpyHostToDevice, (hipStream_t)stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  }
  return decode_enqueue(plan, q, cache, table, params, out, lse, ws, kStaticWorkspaceBytes,
                        stream, true, true);
}

pa_status pa_debug_gather_kv(const pa_kv_cache* cache, const pa_page_table* table,
                             int32_t request, int32_t kv_len, int32_t kv_head, void* k_out,
                             void* v_out, void* stream) {
  pa_status st = check_cache(cache, true);
  if (st != PA_OK) return st;
  if (!table || !table->kv_indptr || !table->kv_indices)
    return fail(PA_ERR_INVALID_ARG, "page table is NULL");
  if (request < 0 || request >= table->batch) return fail(PA_ERR_INVALID_ARG, "request out of range");
  if (kv_head < 0 || kv_head >= cache->num_kv_heads) return fail(PA_ERR_INVALID_ARG, "kv_head out of range");
  if (kv_len < 0) return fail(PA_ERR_INVALID_ARG, "kv_len is negative");
  if (kv_len == 0) return PA_OK;
  if (!k_out || !v_out || (((uintptr_t)k_out | (uintptr_t)v_out) & 15))
    return fail(PA_ERR_INVALID_ARG, "k_out / v_out must be non-NULL and 16-byte aligned");
  const bool fp4 = cache->kv_dtype == PA_DTYPE_NVFP4;
  GatherArgs g;
  g.k = (const char*)cache->k;
  g.v = (const char*)cache->v;
  g.k_sp = cache->k_stride_page; g.k_sh = cache->k_stride_head; g.k_st = cache->k_stride_token;
  g.v_sp = cache->v_stride_page; g.v_sh = cache->v_stride_head; g.v_st = cache->v_stride_token;
  g.k_sf = (const char*)cache->k_sf;
  g.v_sf = (const char*)cache->v_sf;
  g.ks_sp = cache->k_sf_stride_page; g.ks_sh = cache->k_sf_stride_head; g.ks_st = cache->k_sf_stride_token;
  g.vs_sp = cache->v_sf_stride_page; g.vs_sh = cache->v_sf_stride_head; g.vs_st = cache->v_sf_stride_token;
  g.kv_indptr = table->kv_indptr;
  g.kv_indices = table->kv_indices;
  g.b = request;
  g.head = kv_head;
  g.page_size = cache->page_size;
  g.esz = fp4 ? 1 : dtype_bytes(cache->kv_dtype);
  g.k_row_bytes = fp4 ? cache->head_dim_qk / 2 : cache->head_dim_qk * g.esz;
  g.v_row_bytes = fp4 ? cache->head_dim_vo / 2 : cache->head_dim_vo * g.esz;
  g.ks_row_bytes = fp4 ? cache->head_dim_qk / 16 : 0;
  g.vs_row_bytes = fp4 ? cache->head_dim_vo / 16 : 0;
  g.k_out = (char*)k_out;
  g.v_out = (char*)v_out;
  gather_kv_kernel<<<kv_len, 64, 0, (hipStream_t)stream>>>(g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "gather kernel launch: %s", hipGetErrorString(e));
  count_launches(1);
  return PA_OK;
}

pa_status pa_debug_fp8_to_f32(const uint8_t* codes, float* out, int32_t n, void* stream) {
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "n is negative");
  if (n == 0) return PA_OK;
  if (!codes || !out) return fail(PA_ERR_INVALID_ARG, "codes or out is NULL");
  const int threads = (n + 3) / 4;
  fp8_to_f32_kernel<<<(threads + 255) / 256, 256, 0, (hipStream_t)stream>>>(codes, out, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "fp8 kernel launch: %s", hipGetErrorString(e));
  count_launches(1);
  return PA_OK;
}

}  // extern "C"
