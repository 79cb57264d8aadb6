// Internal declarations shared by the host planner (pa_host.cpp) and the HIP launchers.
#pragma once

#include <stdint.h>

#include "pa.h"

namespace pa {

// Decode partition: keys are grouped in logical blocks of 16 tokens (one MFMA tile of
// keys); the work units are (request, KV head, block) triples, and each wave of the
// partial kernel runs a contiguous piece of them.
constexpr int kBlockTokens = 16;
constexpr int kDecodeWaveSlots = 2048;   // 256 CUs x 4 SIMDs x 2 waves (register-bound)
constexpr int kMinPieceBlocks = 8;       // balanced pieces hold at least this many blocks
constexpr int kMaxSplits = 64;
constexpr int kMaxDecodeGroup = 8;       // query heads per KV head in decode
constexpr int kDecodeWavesPerGroup = 8;  // waves per workgroup: the two of every SIMD of a CU
constexpr int kLdsBytesPerCu = 160 * 1024;  // gfx950: LDS of one CU, all of it one workgroup's

// LDS of a decode workgroup (bytes) when its waves keep P buffers of pc columns: per wave
// the group's Q rows (padded pitch), two P and two alpha buffers, its progress word and
// group counter, and a parked split result (G x Dvo outputs and G log-sum-exps); plus a
// margin.  The kernel sizes its buffers with it and the planner decides from it whether
// the kernel can hold split results in LDS.
constexpr int decode_lds_bytes(int dqk, int dvo, int gmax, int pc) {
  return kDecodeWavesPerGroup * (gmax * (dqk + 8) * 2 + 2 * 16 * pc * 4 + 2 * 16 * 4 + 8 +
                                 (gmax * dvo + gmax) * 4) + 1024;
}
// P columns kept: all 16 when they fit, else only those the P V step reads.
constexpr int decode_p_columns(int dqk, int dvo, int gmax, bool fp4) {
  return decode_lds_bytes(dqk, dvo, gmax, 16) <= kLdsBytesPerCu ? 16 : (fp4 ? 8 : gmax);
}
// Whether the decode kernel has an LDS slot per wave for one split result.
constexpr bool decode_parks(int dqk, int dvo, int gmax, bool fp4) {
  return decode_lds_bytes(dqk, dvo, gmax, decode_p_columns(dqk, dvo, gmax, fp4)) <= kLdsBytesPerCu;
}
// Query heads the decode kernel computes for a group of `group` (its instantiations).
constexpr int decode_gmax(int group) { return group <= 4 ? group : group <= 6 ? 6 : 8; }
constexpr int kMaxPrefillGroup = 16;
constexpr int64_t kLastLevelCacheBytes = int64_t(256) << 20;  // MI355X memory-side cache
// NVFP4 prefill widens the table's pages to bf16 once per call when the tiles read each
// key at least this many times on average.
constexpr int64_t kStageMinReads = 4;

// Prefill: query rows per tile ((token, head) pairs of one head group), 16 per wave.
constexpr int kPrefillTileRows = 128;
constexpr int kPrefillWaveRows = 16;
constexpr int kPrefillWaves = kPrefillTileRows / kPrefillWaveRows;
constexpr int kPrefillKeyStage = 32;  // keys per LDS stage of the prefill kernel
// Split-K prefill (a short query over a long KV): when the tiles give fewer than
// kPrefillSplitItems workgroups (tiles x KV heads), tile key ranges longer than the chunk
// length are cut into chunks of whole 32-key stages, chunk length =
// max(kPrefillMinChunkStages, ceil(total stages x KV heads / kPrefillSplitItems)).
constexpr int kPrefillSplitItems = 512;
constexpr int kPrefillMinChunkStages = 8;

// Blocks of one (request, KV head) run by one wave.  The plan holds one head segment per
// wave (index = wave, in launch order), then the waves' further segments; a head segment
// names where its wave's further segments sit, so a wave starts from one record.
struct DecodeSegment {  // 32 bytes
  int32_t b;             // request
  int32_t kvh;           // KV head
  int32_t t_begin;       // first key of the segment
  int32_t t_end;         // one past the last key (t_end > t_begin)
  int32_t slot;          // partial slot, or -1: write the final output directly
  int32_t page_base;     // kv_indptr[b]: the request's first entry in kv_indices
  int32_t more_begin;    // head segments: index of the wave's next segment
  int32_t more_count;    // head segments, bits 0-15: number of further segments of the wave;
                         // the wave's last segment, bits 16-23: size of the group of
                         // neighbouring waves whose results it joins in LDS (0: none),
                         // bits 24-31: that group's first wave within the workgroup
};

struct MergeItem {       // 16 bytes
  int32_t b;
  int32_t kvh;
  int32_t slot_begin;
  int32_t num_slots;     // 0: the request has no keys (zero output, lse -inf)
};

struct PrefillItem {  // 48 bytes
  int32_t b;
  int32_t row_begin;  // first (token, head) row of the tile within the request's group
  int32_t row_end;
  int32_t kv_begin;   // keys this item covers: [kv_begin, kv_end)
  int32_t kv_end;
  int32_t q_begin;    // qo_indptr[b]
  int32_t kv_len;     // L_b
  int32_t q_len;      // qo_indptr[b+1] - qo_indptr[b]
  int32_t slot;       // -1: the tile's whole key range, written to the output; else the
                      // partial slot of one key chunk of a split tile
  int32_t pad[3];
};

// One split tile: its chunks' partials sit in slots [slot_begin, slot_begin + num_slots).
struct PrefillMerge {  // 32 bytes
  int32_t b;
  int32_t row_begin;
  int32_t row_end;
  int32_t q_begin;
  int32_t slot_begin;
  int32_t num_slots;
  int32_t pad[2];
};

pa_status fail(pa_status code, const char* fmt, ...);
void count_launches(uint64_t n);

// Argument checks shared by planning and running.  `need_pointers` also checks the
// cache's base pointers and their alignment.
pa_status check_cache(const pa_kv_cache* c, bool need_pointers);
pa_status check_params(const pa_attn_params* p, const pa_kv_cache* c, int max_group);
pa_status check_plan_matches(const pa_plan* plan, int kind, const pa_attn_params* p,
                             const pa_kv_cache* c, const pa_page_table* t,
                             size_t workspace_bytes);

inline int dtype_bytes(int32_t dt) { return dt == PA_DTYPE_FP8_E4M3FN ? 1 : (dt == PA_DTYPE_FP32 ? 4 : 2); }

}  // namespace pa
