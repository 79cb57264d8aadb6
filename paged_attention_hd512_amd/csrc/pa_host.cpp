// Host half of libpa: error state, cache descriptors, validation and the work planners.
// Nothing in this file calls HIP, so every function here runs on a machine without a GPU.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <string>
#include <vector>

#include "pa_internal.hpp"

namespace pa {

static thread_local std::string g_last_error;
static std::atomic<uint64_t> g_launches{0};

pa_status fail(pa_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void count_launches(uint64_t n) { g_launches.fetch_add(n, std::memory_order_relaxed); }

static bool supported_dims(int qk, int vo) {
  return (qk == 512 && vo == 512) || (qk == 256 && vo == 256) || (qk == 512 && vo == 256);
}

pa_status check_cache(const pa_kv_cache* c, bool need_pointers) {
  if (!c) return fail(PA_ERR_INVALID_ARG, "cache is NULL");
  if (c->kv_dtype != PA_DTYPE_BF16 && c->kv_dtype != PA_DTYPE_FP8_E4M3FN &&
      c->kv_dtype != PA_DTYPE_NVFP4)
    return fail(PA_ERR_UNSUPPORTED, "kv_dtype %d: only bf16, fp8 e4m3fn and nvfp4 KV are supported",
                c->kv_dtype);
  const bool fp4 = c->kv_dtype == PA_DTYPE_NVFP4;
  // A block-scale tensor on a cache that is not NVFP4 is refused rather than ignored (the
  // FlashInfer page's review on output sizing keyed on a stray scale-factor tensor).
  if (!fp4 && (c->k_sf || c->v_sf))
    return fail(PA_ERR_INVALID_ARG, "k_sf / v_sf are set on a cache whose kv_dtype is not nvfp4");
  if (c->num_pages < 1 || c->num_kv_heads < 1 || c->page_size < 1)
    return fail(PA_ERR_INVALID_ARG, "num_pages (%d), num_kv_heads (%d) and page_size (%d) must be >= 1",
                c->num_pages, c->num_kv_heads, c->page_size);
  if (!supported_dims(c->head_dim_qk, c->head_dim_vo))
    return fail(PA_ERR_UNSUPPORTED,
                "head dims (qk=%d, vo=%d): supported are (512,512), (256,256), (512,256)",
                c->head_dim_qk, c->head_dim_vo);
  // Stored units per 16-byte vector: elements, or bytes for NVFP4 (two elements each).
  const int64_t vec = fp4 ? 16 : 16 / dtype_bytes(c->kv_dtype);
  const int64_t s[6] = {c->k_stride_page, c->k_stride_head, c->k_stride_token,
                        c->v_stride_page, c->v_stride_head, c->v_stride_token};
  const char* names[6] = {"k_stride_page", "k_stride_head", "k_stride_token",
                          "v_stride_page", "v_stride_head", "v_stride_token"};
  for (int i = 0; i < 6; ++i) {
    if (s[i] < 0) return fail(PA_ERR_INVALID_ARG, "%s is negative", names[i]);
    if (s[i] % vec)
      return fail(PA_ERR_UNSUPPORTED, "%s = %lld is not a multiple of 16 bytes", names[i],
                  (long long)s[i]);
  }
  if (fp4) {
    const int64_t f[6] = {c->k_sf_stride_page, c->k_sf_stride_head, c->k_sf_stride_token,
                          c->v_sf_stride_page, c->v_sf_stride_head, c->v_sf_stride_token};
    const char* fn[6] = {"k_sf_stride_page", "k_sf_stride_head", "k_sf_stride_token",
                         "v_sf_stride_page", "v_sf_stride_head", "v_sf_stride_token"};
    for (int i = 0; i < 6; ++i) {
      if (f[i] < 0) return fail(PA_ERR_INVALID_ARG, "%s is negative", fn[i]);
      if (f[i] % 16)
        return fail(PA_ERR_UNSUPPORTED, "%s = %lld is not a multiple of 16 bytes", fn[i],
                    (long long)f[i]);
    }
  }
  if (c->kv_dtype == PA_DTYPE_BF16 && (c->k_scale != 1.0f || c->v_scale != 1.0f))
    return fail(PA_ERR_INVALID_ARG, "bf16 KV takes k_scale = v_scale = 1");
  if (!(std::isfinite(c->k_scale) && c->k_scale > 0.f && std::isfinite(c->v_scale) &&
        c->v_scale > 0.f))
    return fail(PA_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if (need_pointers) {
    if (!c->k || !c->v) return fail(PA_ERR_INVALID_ARG, "cache k/v pointer is NULL");
    if (((uintptr_t)c->k | (uintptr_t)c->v) & 15)
      return fail(PA_ERR_UNSUPPORTED, "cache k/v pointers must be 16-byte aligned");
    if (fp4) {
      if (!c->k_sf || !c->v_sf) return fail(PA_ERR_INVALID_ARG, "nvfp4 cache: k_sf / v_sf is NULL");
      if (((uintptr_t)c->k_sf | (uintptr_t)c->v_sf) & 15)
        return fail(PA_ERR_UNSUPPORTED, "nvfp4 cache: k_sf / v_sf must be 16-byte aligned");
    }
  }
  return PA_OK;
}

pa_status check_params(const pa_attn_params* p, const pa_kv_cache* c, int max_group) {
  if (!p) return fail(PA_ERR_INVALID_ARG, "params is NULL");
  if (p->num_qo_heads < 1) return fail(PA_ERR_INVALID_ARG, "num_qo_heads must be >= 1");
  if (p->num_qo_heads % c->num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "num_qo_heads (%d) is not a multiple of num_kv_heads (%d)",
                p->num_qo_heads, c->num_kv_heads);
  const int group = p->num_qo_heads / c->num_kv_heads;
  if (group > max_group)
    return fail(PA_ERR_UNSUPPORTED, "%d query heads per KV head; at most %d are supported",
                group, max_group);
  if (!std::isfinite(p->sm_scale)) return fail(PA_ERR_INVALID_ARG, "sm_scale is not finite");
  if (p->q_dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_UNSUPPORTED, "q_dtype %d: only bf16 queries are supported", p->q_dtype);
  if (p->out_dtype != PA_DTYPE_BF16 && p->out_dtype != PA_DTYPE_FP32)
    return fail(PA_ERR_UNSUPPORTED, "out_dtype %d: only fp32 and bf16 outputs are supported",
                p->out_dtype);
  return PA_OK;
}

static int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

static pa_status check_table_host(const int32_t* indptr, const int32_t* last, int32_t batch,
                                  int32_t page_size) {
  if (batch < 0) return fail(PA_ERR_INVALID_ARG, "batch is negative");
  if (batch == 0) return PA_OK;
  if (!indptr || !last) return fail(PA_ERR_INVALID_ARG, "host kv_indptr / kv_last_page_len is NULL");
  if (indptr[0] != 0) return fail(PA_ERR_INVALID_ARG, "kv_indptr[0] = %d, must be 0", indptr[0]);
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t n = indptr[b + 1] - indptr[b];
    if (n < 0) return fail(PA_ERR_INVALID_ARG, "kv_indptr decreases at request %d", b);
    if (n > 0 && (last[b] < 1 || last[b] > page_size))
      return fail(PA_ERR_INVALID_ARG, "kv_last_page_len[%d] = %d is outside [1, %d]", b, last[b],
                  page_size);
    const int64_t len = n == 0 ? 0 : (int64_t)(n - 1) * page_size + last[b];
    if (len > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "request %d is longer than 2^31 keys", b);
  }
  return PA_OK;
}

static int64_t kv_len_of(const int32_t* indptr, const int32_t* last, int32_t b, int32_t page_size) {
  const int32_t n = indptr[b + 1] - indptr[b];
  return n == 0 ? 0 : (int64_t)(n - 1) * page_size + last[b];
}

static void plan_header(pa_plan* plan, int kind, const pa_attn_params* p, const pa_kv_cache* c,
                        int32_t batch) {
  memset(plan, 0, sizeof(*plan));
  plan->kind = kind;
  plan->batch = batch;
  plan->num_qo_heads = p->num_qo_heads;
  plan->num_kv_heads = c->num_kv_heads;
  plan->page_size = c->page_size;
  plan->head_dim_qk = c->head_dim_qk;
  plan->head_dim_vo = c->head_dim_vo;
  plan->kv_dtype = c->kv_dtype;
  plan->window = p->window > 0 ? p->window : 0;
  plan->causal = p->causal ? 1 : 0;
}

pa_status check_plan_matches(const pa_plan* plan, int kind, const pa_attn_params* p,
                             const pa_kv_cache* c, const pa_page_table* t,
                             size_t workspace_bytes) {
  if (!plan) return fail(PA_ERR_INVALID_ARG, "plan is NULL");
  if (!t) return fail(PA_ERR_INVALID_ARG, "page table is NULL");
  if (plan->kind != kind) return fail(PA_ERR_INVALID_ARG, "plan kind %d does not match this call", plan->kind);
  const int window = p->window > 0 ? p->window : 0;
  if (plan->batch != t->batch || plan->num_qo_heads != p->num_qo_heads ||
      plan->num_kv_heads != c->num_kv_heads || plan->page_size != c->page_size ||
      plan->head_dim_qk != c->head_dim_qk || plan->head_dim_vo != c->head_dim_vo ||
      plan->kv_dtype != c->kv_dtype || plan->window != window ||
      (kind == 2 && plan->causal != (p->causal ? 1 : 0)))
    return fail(PA_ERR_INVALID_ARG,
                "plan was made for other sizes (batch, heads, page size, head dims, dtype, "
                "window or causal differ)");
  if ((int64_t)workspace_bytes < plan->workspace_bytes)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, plan needs %lld",
                workspace_bytes, (long long)plan->workspace_bytes);
  if (t->batch > 0 && (!t->kv_indptr || !t->kv_indices || !t->kv_last_page_len))
    return fail(PA_ERR_INVALID_ARG, "device page table pointer is NULL");
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" {

const char* pa_last_error(void) { return g_last_error.c_str(); }
uint64_t pa_launch_count(void) { return g_launches.load(std::memory_order_relaxed); }
uint64_t pa_debug_launch_count(void) { return pa_launch_count(); }
const char* pa_version(void) { return "libpa 0.1.0 (gfx950)"; }

pa_status pa_kv_cache_hnd(const void* base, int32_t kv_dtype, int32_t num_pages,
                          int32_t num_kv_heads, int32_t page_size, int32_t head_dim,
                          float k_scale, float v_scale, pa_kv_cache* out) {
  if (!out) return fail(PA_ERR_INVALID_ARG, "out is NULL");
  if (kv_dtype == PA_DTYPE_NVFP4)
    return fail(PA_ERR_INVALID_ARG, "nvfp4 caches carry block scales: use pa_kv_cache_nvfp4_hnd");
  pa_kv_cache c;
  memset(&c, 0, sizeof(c));
  const int esz = dtype_bytes(kv_dtype);
  c.k = base;
  c.v = base ? (const void*)((const char*)base + (size_t)num_kv_heads * page_size * head_dim * esz)
             : nullptr;
  c.kv_dtype = kv_dtype;
  c.num_pages = num_pages;
  c.num_kv_heads = num_kv_heads;
  c.page_size = page_size;
  c.head_dim_qk = c.head_dim_vo = head_dim;
  c.k_stride_token = c.v_stride_token = head_dim;
  c.k_stride_head = c.v_stride_head = (int64_t)page_size * head_dim;
  c.k_stride_page = c.v_stride_page = 2 * (int64_t)num_kv_heads * page_size * head_dim;
  c.k_scale = k_scale;
  c.v_scale = v_scale;
  pa_status st = check_cache(&c, false);
  if (st != PA_OK) return st;
  *out = c;
  return PA_OK;
}

pa_status pa_kv_cache_separate(const void* k, const void* v, int32_t kv_dtype,
                               int32_t num_pages, int32_t num_kv_heads, int32_t page_size,
                               int32_t head_dim_qk, int32_t head_dim_vo, float k_scale,
                               float v_scale, pa_kv_cache* out) {
  if (!out) return fail(PA_ERR_INVALID_ARG, "out is NULL");
  if (kv_dtype == PA_DTYPE_NVFP4)
    return fail(PA_ERR_INVALID_ARG,
                "nvfp4 caches carry block scales: use pa_kv_cache_nvfp4_separate");
  pa_kv_cache c;
  memset(&c, 0, sizeof(c));
  c.k = k;
  c.v = v;
  c.kv_dtype = kv_dtype;
  c.num_pages = num_pages;
  c.num_kv_heads = num_kv_heads;
  c.page_size = page_size;
  c.head_dim_qk = head_dim_qk;
  c.head_dim_vo = head_dim_vo;
  c.k_stride_token = head_dim_qk;
  c.k_stride_head = (int64_t)page_size * head_dim_qk;
  c.k_stride_page = (int64_t)num_kv_heads * page_size * head_dim_qk;
  c.v_stride_token = head_dim_vo;
  c.v_stride_head = (int64_t)page_size * head_dim_vo;
  c.v_stride_page = (int64_t)num_kv_heads * page_size * head_dim_vo;
  c.k_scale = k_scale;
  c.v_scale = v_scale;
  pa_status st = check_cache(&c, false);
  if (st != PA_OK) return st;
  *out = c;
  return PA_OK;
}

pa_status pa_kv_cache_nvfp4_separate(const void* k, const void* v, const void* k_sf,
                                     const void* v_sf, int32_t num_pages,
                                     int32_t num_kv_heads, int32_t page_size,
                                     int32_t head_dim_qk, int32_t head_dim_vo, float k_scale,
                                     float v_scale, pa_kv_cache* out) {
  if (!out) return fail(PA_ERR_INVALID_ARG, "out is NULL");
  pa_kv_cache c;
  memset(&c, 0, sizeof(c));
  c.k = k;
  c.v = v;
  c.k_sf = k_sf;
  c.v_sf = v_sf;
  c.kv_dtype = PA_DTYPE_NVFP4;
  c.num_pages = num_pages;
  c.num_kv_heads = num_kv_heads;
  c.page_size = page_size;
  c.head_dim_qk = head_dim_qk;
  c.head_dim_vo = head_dim_vo;
  const int64_t kb = head_dim_qk / 2, vb = head_dim_vo / 2;      // data bytes per row
  const int64_t kf = head_dim_qk / 16, vf = head_dim_vo / 16;    // block scales per row
  c.k_stride_token = kb;
  c.k_stride_head = (int64_t)page_size * kb;
  c.k_stride_page = (int64_t)num_kv_heads * page_size * kb;
  c.v_stride_token = vb;
  c.v_stride_head = (int64_t)page_size * vb;
  c.v_stride_page = (int64_t)num_kv_heads * page_size * vb;
  c.k_sf_stride_token = kf;
  c.k_sf_stride_head = (int64_t)page_size * kf;
  c.k_sf_stride_page = (int64_t)num_kv_heads * page_size * kf;
  c.v_sf_stride_token = vf;
  c.v_sf_stride_head = (int64_t)page_size * vf;
  c.v_sf_stride_page = (int64_t)num_kv_heads * page_size * vf;
  c.k_scale = k_scale;
  c.v_scale = v_scale;
  pa_status st = check_cache(&c, false);
  if (st != PA_OK) return st;
  *out = c;
  return PA_OK;
}

pa_status pa_kv_cache_nvfp4_hnd(const void* data, const void* sf, int32_t num_pages,
                                int32_t num_kv_heads, int32_t page_size, int32_t head_dim,
                                float k_scale, float v_scale, pa_kv_cache* out) {
  if (!out) return fail(PA_ERR_INVALID_ARG, "out is NULL");
  const int64_t half_d = (int64_t)num_kv_heads * page_size * (head_dim / 2);    // K half, bytes
  const int64_t half_f = (int64_t)num_kv_heads * page_size * (head_dim / 16);
  const char* d = (const char*)data;
  const char* f = (const char*)sf;
  pa_status st = pa_kv_cache_nvfp4_separate(d, d ? d + half_d : nullptr, f, f ? f + half_f : nullptr,
                                            num_pages, num_kv_heads, page_size, head_dim,
                                            head_dim, k_scale, v_scale, out);
  if (st != PA_OK) return st;
  out->k_stride_page = out->v_stride_page = 2 * half_d;
  out->k_sf_stride_page = out->v_sf_stride_page = 2 * half_f;
  return check_cache(out, false);
}

pa_status pa_validate_page_table_host(const int32_t* kv_indptr_host,
                                      const int32_t* kv_indices_host,
                                      const int32_t* kv_last_page_len_host, int32_t batch,
                                      int32_t num_pages, int32_t page_size) {
  if (page_size < 1) return fail(PA_ERR_INVALID_ARG, "page_size must be >= 1");
  pa_status st = check_table_host(kv_indptr_host, kv_last_page_len_host, batch, page_size);
  if (st != PA_OK || batch == 0 || !kv_indices_host) return st;
  const int32_t n = kv_indptr_host[batch];
  for (int32_t i = 0; i < n; ++i)
    if (kv_indices_host[i] < 0 || kv_indices_host[i] >= num_pages)
      return fail(PA_ERR_INVALID_ARG, "kv_indices[%d] = %d is outside [0, %d)", i,
                  kv_indices_host[i], num_pages);
  return PA_OK;
}

pa_status pa_decode_plan(const pa_attn_params* params, const pa_kv_cache* cache,
                         const int32_t* kv_indptr_host, const int32_t* kv_last_page_len_host,
                         int32_t batch, int32_t num_splits, void* plan_buf_host,
                         size_t plan_buf_bytes, pa_plan* plan) {
  if (!plan) return fail(PA_ERR_INVALID_ARG, "plan is NULL");
  pa_status st = check_cache(cache, false);
  if (st != PA_OK) return st;
  if ((st = check_params(params, cache, kMaxDecodeGroup)) != PA_OK) return st;
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(PA_ERR_UNSUPPORTED, "num_splits = %d: must be in [0, %d] (0 = adaptive)",
                num_splits, kMaxSplits);
  if ((st = check_table_host(kv_indptr_host, kv_last_page_len_host, batch, cache->page_size)) != PA_OK)
    return st;

  const int window = params->window > 0 ? params->window : 0;
  const int P = cache->page_size;
  const int32_t hkv = cache->num_kv_heads;
  std::vector<int64_t> len(batch), start(batch), nblk(batch);
  int64_t max_len = 0;
  for (int32_t b = 0; b < batch; ++b) {
    len[b] = kv_len_of(kv_indptr_host, kv_last_page_len_host, b, P);
    start[b] = window > 0 ? std::max<int64_t>(0, len[b] - window) : 0;
    const int64_t fb = start[b] / kBlockTokens;
    const int64_t eb = (len[b] + kBlockTokens - 1) / kBlockTokens;
    nblk[b] = std::max<int64_t>(0, eb - fb);
    max_len = std::max(max_len, len[b]);
  }
  // Flattened units: (b, h, block) in that order; pair i = b * hkv + h starts at origin[i].
  const int64_t npairs = (int64_t)batch * hkv;
  std::vector<int64_t> origin(npairs + 1);
  origin[0] = 0;
  for (int64_t i = 0; i < npairs; ++i) origin[i + 1] = origin[i] + nblk[i / hkv];
  const int64_t total = origin[npairs];

  // Pieces (one wave each): the flattened axis in near-equal parts.
  std::vector<std::pair<int64_t, int64_t>> pieces;
  {
    // The largest piece sets the launch's length, and while the waves with one block more
    // than the rest finish, the others leave HBM idle: keep the largest size that
    // min(wave slots, units / 8) pieces would need, and use as few pieces as that size
    // allows, so (nearly) every piece holds it.
    const int64_t np0 = std::min<int64_t>(kDecodeWaveSlots, (total + kMinPieceBlocks - 1) / kMinPieceBlocks);
    const int64_t per = np0 > 0 ? (total + np0 - 1) / np0 : 0;
    const int64_t np = per > 0 ? (total + per - 1) / per : 0;
    // Without a fixed split, when cutting each (b, h) on its own into near-equal pieces of
    // at most that size takes no more waves than there are slots, no piece crosses a pair
    // boundary: every wave then runs one segment, and none pays a second start.
    int64_t aligned = 0;
    for (int64_t i = 0; i < npairs; ++i) aligned += (origin[i + 1] - origin[i] + per - 1) / std::max<int64_t>(per, 1);
    if (num_splits == 0 && per > 0 && aligned <= kDecodeWaveSlots) {
      for (int64_t i = 0; i < npairs; ++i) {
        const int64_t n = origin[i + 1] - origin[i];
        const int64_t c = (n + per - 1) / per;
        for (int64_t k = 0; k < c; ++k) pieces.emplace_back(origin[i] + n * k / c, origin[i] + n * (k + 1) / c);
      }
    } else {
      for (int64_t k = 0; k < np; ++k) pieces.emplace_back(total * k / np, total * (k + 1) / np);
    }
  }
  // End of the segment that starts at unit u of pair i: the pair's end, or with a fixed
  // split S the next of the S chunk boundaries of the pair, [o + n k / c) with c = min(S, n).
  auto segment_end = [&](int64_t i, int64_t u) {
    int64_t e = origin[i + 1];
    if (num_splits > 0) {
      const int64_t n = origin[i + 1] - origin[i];
      const int64_t c = std::min<int64_t>(num_splits, n);
      for (int64_t k = 1; k < c; ++k) {
        const int64_t cut = origin[i] + n * k / c;
        if (cut > u) {
          e = cut;
          break;
        }
      }
    }
    return e;
  };

  // Cut each piece into segments at (b, h) boundaries (and fixed-split chunk boundaries);
  // pieces run in flattened order, so the pair index only moves forward.
  std::vector<std::vector<DecodeSegment>> piece_segs(pieces.size());
  std::vector<int32_t> seg_count(npairs, 0);
  int64_t pair = 0;
  for (size_t k = 0; k < pieces.size(); ++k) {
    int64_t u = pieces[k].first;
    const int64_t u1 = pieces[k].second;
    while (u < u1) {
      while (origin[pair + 1] <= u) ++pair;  // skips empty ranges too
      const int32_t b = (int32_t)(pair / hkv), h = (int32_t)(pair % hkv);
      const int64_t e = std::min<int64_t>(u1, segment_end(pair, u));
      const int64_t fb = start[b] / kBlockTokens;
      const int64_t t0 = std::max<int64_t>(start[b], (fb + u - origin[pair]) * kBlockTokens);
      const int64_t t1 = std::min<int64_t>(len[b], (fb + e - origin[pair]) * kBlockTokens);
      DecodeSegment sg;
      memset(&sg, 0, sizeof(sg));
      sg.b = b; sg.kvh = h; sg.t_begin = (int32_t)t0; sg.t_end = (int32_t)t1; sg.slot = -1;
      sg.page_base = kv_indptr_host[b];
      piece_segs[k].push_back(sg);
      ++seg_count[pair];
      u = e;
    }
  }
  // Launch order: longest piece first, ties in piece order.
  std::vector<int32_t> order(pieces.size());
  for (size_t k = 0; k < order.size(); ++k) order[k] = (int32_t)k;
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    return pieces[x].second - pieces[x].first > pieces[y].second - pieces[y].first;
  });
  // Grouped split results: where the kernel holds split results in LDS, the last segments
  // of consecutive waves of one workgroup (launch order, kDecodeWavesPerGroup waves each)
  // that belong to one split (b, h) form a group; the last of its waves to finish combines
  // the group's results and writes one partial.  grp_lead[k] is the group's first piece in
  // launch order (-1: piece k's last segment is in no group).
  const bool group_last = decode_parks(cache->head_dim_qk, cache->head_dim_vo,
                                       decode_gmax(params->num_qo_heads / hkv),
                                       cache->kv_dtype == PA_DTYPE_NVFP4);
  std::vector<int32_t> grp_lead(pieces.size(), -1), grp_pos(pieces.size(), 0), grp_size(pieces.size(), 0);
  if (group_last) {
    const size_t np = order.size();
    auto last_pair = [&](size_t s) {
      const DecodeSegment& L = piece_segs[order[s]].back();
      return (int64_t)L.b * hkv + L.kvh;
    };
    for (size_t s = 0; s < np;) {
      const int64_t i = last_pair(s);
      size_t e = s + 1;
      if (seg_count[i] > 1)
        while (e < np && e / kDecodeWavesPerGroup == s / kDecodeWavesPerGroup && last_pair(e) == i) ++e;
      if (e - s >= 2)
        for (size_t t = s; t < e; ++t) {
          grp_lead[order[t]] = order[s];
          grp_pos[order[t]] = (int32_t)(s % kDecodeWavesPerGroup);
          grp_size[order[t]] = (int32_t)(e - s);
        }
      s = e;
    }
  }
  // Slots, numbered in (b, h) order; within a (b, h), one per segment (one per group for
  // grouped segments), in piece order.  Merge entries for split and for empty pairs.
  std::vector<int32_t> units(npairs, 0);
  for (size_t k = 0; k < piece_segs.size(); ++k)
    for (size_t j = 0; j < piece_segs[k].size(); ++j) {
      const DecodeSegment& sg = piece_segs[k][j];
      const int64_t i = (int64_t)sg.b * hkv + sg.kvh;
      const bool grouped = j + 1 == piece_segs[k].size() && grp_lead[k] >= 0;
      if (seg_count[i] > 1 && (!grouped || grp_lead[k] == (int32_t)k)) ++units[i];
    }
  std::vector<int32_t> first_slot(npairs, -1);
  std::vector<MergeItem> merges;
  int32_t next_slot = 0;
  for (int64_t i = 0; i < npairs; ++i) {
    const int32_t b = (int32_t)(i / hkv), h = (int32_t)(i % hkv);
    if (seg_count[i] == 0) {
      merges.push_back(MergeItem{b, h, next_slot, 0});
    } else if (seg_count[i] > 1) {
      first_slot[i] = next_slot;
      merges.push_back(MergeItem{b, h, next_slot, units[i]});
      next_slot += units[i];
    }
  }
  std::vector<int32_t> used(npairs, 0), grp_slot(pieces.size(), -1);
  for (size_t k = 0; k < piece_segs.size(); ++k)
    for (size_t j = 0; j < piece_segs[k].size(); ++j) {
      DecodeSegment& sg = piece_segs[k][j];
      const int64_t i = (int64_t)sg.b * hkv + sg.kvh;
      if (first_slot[i] < 0) continue;
      if (j + 1 == piece_segs[k].size() && grp_lead[k] >= 0) {
        int32_t& gs = grp_slot[grp_lead[k]];
        if (gs < 0) gs = first_slot[i] + used[i]++;
        sg.slot = gs;
      } else {
        sg.slot = first_slot[i] + used[i]++;
      }
    }
  int64_t num_segs = 0;
  for (auto& segs : piece_segs) {
    // A wave's record counts its further segments in 16 bits (the bits above carry its group).
    if (segs.size() > 0x10000)
      return fail(PA_ERR_UNSUPPORTED, "a wave would run %zu segments; at most 65536 are supported",
                  segs.size());
    num_segs += (int64_t)segs.size();
  }
  if (num_segs > INT32_MAX / 2) return fail(PA_ERR_UNSUPPORTED, "too many decode segments");

  plan_header(plan, 1, params, cache, batch);
  plan->num_items = (int32_t)num_segs;
  plan->num_workers = (int32_t)pieces.size();
  plan->num_slots = next_slot;
  plan->num_merges = (int32_t)merges.size();
  plan->block_tokens = kBlockTokens;
  plan->chunk_blocks = pieces.empty() ? 0 : (int32_t)(pieces[order[0]].second - pieces[order[0]].first);
  plan->num_splits = num_splits;
  plan->max_kv_len = (int32_t)max_len;
  // Waves that finish a split segment before their last one would store its result while
  // their next segment streams.  Such stores in a quarter or more of the waves slowed every
  // wave's reads (GQA batch at split-K 8, 46 % of the waves: 226 -> 206 us when the results
  // wait in LDS until the wave ends); with an eighth of the waves the wait cost ~1 % (FP8
  // batch), so the kernel parks them only when they are common.
  int64_t mid_partials = 0;
  for (auto& segs : piece_segs) {
    bool any = false;
    for (size_t k = 0; k + 1 < segs.size(); ++k) any = any || segs[k].slot >= 0;
    mid_partials += any ? 1 : 0;
  }
  plan->deferred_partials = 4 * mid_partials >= (int64_t)pieces.size() && !pieces.empty() ? 1 : 0;
  plan->grouped_partials = group_last ? 1 : 0;
  // Segments: the head segment of every wave (in launch order), then the further segments
  // of the waves that have several (workers_offset), wave after wave.
  plan->items_offset = 0;
  plan->workers_offset = (int64_t)pieces.size() * (int64_t)sizeof(DecodeSegment);
  plan->merges_offset = align_up(num_segs * (int64_t)sizeof(DecodeSegment), 16);
  plan->plan_bytes = align_up(plan->merges_offset + (int64_t)merges.size() * sizeof(MergeItem), 256);
  plan->partial_o_offset = plan->plan_bytes;
  const int32_t group = params->num_qo_heads / hkv;
  const int64_t o_bytes = (int64_t)next_slot * group * cache->head_dim_vo * 4;
  plan->partial_lse_offset = align_up(plan->partial_o_offset + o_bytes, 256);
  plan->workspace_bytes = align_up(plan->partial_lse_offset + (int64_t)next_slot * group * 4, 256);

  if (!plan_buf_host) return PA_OK;  // sizing call
  if ((int64_t)plan_buf_bytes < plan->plan_bytes)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "plan buffer has %zu bytes, plan needs %lld",
                plan_buf_bytes, (long long)plan->plan_bytes);
  char* buf = (char*)plan_buf_host;
  memset(buf, 0, (size_t)plan->plan_bytes);
  DecodeSegment* out_segs = (DecodeSegment*)(buf + plan->items_offset);
  int32_t more = (int32_t)order.size();  // next free index after the head segments
  for (size_t w = 0; w < order.size(); ++w) {
    const int32_t k0 = order[w];
    const std::vector<DecodeSegment>& segs = piece_segs[k0];
    // The wave's last segment carries its group (more_count bits 16-23: size, 24-31: the
    // group's first wave within the workgroup).
    const int32_t gbits = grp_lead[k0] >= 0 ? (grp_size[k0] << 16) | (grp_pos[k0] << 24) : 0;
    DecodeSegment head = segs[0];
    head.more_begin = more;
    head.more_count = (int32_t)segs.size() - 1;
    if (segs.size() == 1) head.more_count |= gbits;
    out_segs[w] = head;
    for (size_t k = 1; k < segs.size(); ++k) {
      DecodeSegment sg = segs[k];
      if (k + 1 == segs.size()) sg.more_count |= gbits;
      out_segs[more++] = sg;
    }
  }
  if (!merges.empty())
    memcpy(buf + plan->merges_offset, merges.data(), merges.size() * sizeof(MergeItem));
  return PA_OK;
}

pa_status pa_prefill_plan(const pa_attn_params* params, const pa_kv_cache* cache,
                          const int32_t* qo_indptr_host, const int32_t* kv_indptr_host,
                          const int32_t* kv_last_page_len_host, int32_t batch,
                          void* plan_buf_host, size_t plan_buf_bytes, pa_plan* plan) {
  if (!plan) return fail(PA_ERR_INVALID_ARG, "plan is NULL");
  pa_status st = check_cache(cache, false);
  if (st != PA_OK) return st;
  if ((st = check_params(params, cache, kMaxPrefillGroup)) != PA_OK) return st;
  if ((st = check_table_host(kv_indptr_host, kv_last_page_len_host, batch, cache->page_size)) != PA_OK)
    return st;
  if (batch > 0) {
    if (!qo_indptr_host) return fail(PA_ERR_INVALID_ARG, "host qo_indptr is NULL");
    if (qo_indptr_host[0] != 0) return fail(PA_ERR_INVALID_ARG, "qo_indptr[0] must be 0");
  }
  const int P = cache->page_size;
  const int group = params->num_qo_heads / cache->num_kv_heads;
  const int window = params->window > 0 ? params->window : 0;
  const bool causal = params->causal != 0;
  struct Tmp { PrefillItem it; int32_t j; };
  std::vector<Tmp> tiles;
  int64_t max_len = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t q_len = (int64_t)qo_indptr_host[b + 1] - qo_indptr_host[b];
    if (q_len < 0) return fail(PA_ERR_INVALID_ARG, "qo_indptr decreases at request %d", b);
    const int64_t L = kv_len_of(kv_indptr_host, kv_last_page_len_host, b, P);
    if (q_len > L)
      return fail(PA_ERR_INVALID_ARG, "request %d has %lld new tokens but only %lld keys", b,
                  (long long)q_len, (long long)L);
    max_len = std::max(max_len, L);
    const int64_t rows = q_len * group;
    if (rows > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "request %d has too many query rows", b);
    int32_t j = 0;
    for (int64_t r0 = 0; r0 < rows; r0 += kPrefillTileRows, ++j) {
      const int64_t r1 = std::min<int64_t>(rows, r0 + kPrefillTileRows);
      const int64_t pos_first = L - q_len + r0 / group;
      const int64_t pos_last = L - q_len + (r1 - 1) / group;
      const int64_t kv_end = causal ? pos_last + 1 : L;
      const int64_t kv_begin = window > 0 ? std::max<int64_t>(0, pos_first - window + 1) : 0;
      PrefillItem it;
      memset(&it, 0, sizeof(it));
      it.b = b; it.row_begin = (int32_t)r0; it.row_end = (int32_t)r1;
      it.kv_begin = (int32_t)kv_begin; it.kv_end = (int32_t)kv_end;
      it.q_begin = qo_indptr_host[b]; it.kv_len = (int32_t)L; it.q_len = (int32_t)q_len;
      it.slot = -1;
      tiles.push_back(Tmp{it, j});
    }
  }
  // Split-K (a short query over a long KV): with fewer than kPrefillSplitItems workgroups,
  // tile key ranges longer than `chunk` stages are cut into ceil(stages / chunk) near-equal
  // runs of whole stages; each chunk writes a partial to its own slot (slots numbered in
  // tile order) and the tile gets a merge entry.
  const int64_t hkv = cache->num_kv_heads;
  auto stages_of = [](const PrefillItem& it) -> int64_t {
    return it.kv_end > it.kv_begin
               ? (it.kv_end + kPrefillKeyStage - 1) / kPrefillKeyStage - it.kv_begin / kPrefillKeyStage
               : 0;
  };
  int64_t chunk = 0;
  if ((int64_t)tiles.size() * hkv < kPrefillSplitItems) {
    int64_t total = 0;
    for (const Tmp& t : tiles) total += stages_of(t.it);
    chunk = std::max<int64_t>(kPrefillMinChunkStages,
                              (total * hkv + kPrefillSplitItems - 1) / kPrefillSplitItems);
  }
  std::vector<Tmp> items;
  std::vector<PrefillMerge> merges;
  int64_t num_slots = 0;
  for (const Tmp& t : tiles) {
    const int64_t s = stages_of(t.it);
    if (chunk == 0 || s <= chunk) {
      items.push_back(t);
      continue;
    }
    const int64_t c = (s + chunk - 1) / chunk;
    PrefillMerge m;
    memset(&m, 0, sizeof(m));
    m.b = t.it.b; m.row_begin = t.it.row_begin; m.row_end = t.it.row_end;
    m.q_begin = t.it.q_begin; m.slot_begin = (int32_t)num_slots; m.num_slots = (int32_t)c;
    merges.push_back(m);
    const int64_t s0 = t.it.kv_begin / kPrefillKeyStage;
    for (int64_t k = 0; k < c; ++k) {
      Tmp u = t;
      u.it.kv_begin = (int32_t)std::max<int64_t>(t.it.kv_begin, (s0 + s * k / c) * kPrefillKeyStage);
      u.it.kv_end = (int32_t)std::min<int64_t>(t.it.kv_end, (s0 + s * (k + 1) / c) * kPrefillKeyStage);
      u.it.slot = (int32_t)num_slots++;
      items.push_back(u);
    }
  }
  if (num_slots > INT32_MAX / 2) return fail(PA_ERR_UNSUPPORTED, "too many prefill partials");
  std::stable_sort(items.begin(), items.end(), [](const Tmp& a, const Tmp& b) {
    return (a.it.kv_end - a.it.kv_begin) > (b.it.kv_end - b.it.kv_begin);
  });
  // NVFP4 without split-K: when the tiles read every key several times, widening each page
  // once per call (to bf16, in the workspace) costs less than widening each key in every
  // tile that reads it; the bf16 kernel then runs over the widened pages.
  int64_t staged_pages = 0;
  if (cache->kv_dtype == PA_DTYPE_NVFP4 && chunk == 0 && !items.empty() && batch > 0) {
    int64_t reads = 0;
    for (const Tmp& t : items) reads += t.it.kv_end - t.it.kv_begin;
    const int64_t entries = kv_indptr_host[batch];
    if (entries > 0 && reads >= kStageMinReads * entries * cache->page_size) staged_pages = entries;
  }
  // Without split-K, when the K and V bytes the tiles read do not fit the last-level cache,
  // the tiles run request by request (requests in the order of their longest tile, key
  // count descending within each): the tiles running together then read one request's keys,
  // which stay in that cache for the tiles that start later.
  if (chunk == 0 && !items.empty()) {
    const int64_t dk = cache->head_dim_qk + cache->head_dim_vo;
    const int64_t per_key = cache->kv_dtype == PA_DTYPE_BF16 || staged_pages > 0 ? 2 * dk
                            : cache->kv_dtype == PA_DTYPE_NVFP4 ? dk / 2 + dk / 16
                                                                : dk;  // FP8
    std::vector<int64_t> lo(batch, INT64_MAX), hi(batch, INT64_MIN);
    for (const Tmp& t : items) {
      lo[t.it.b] = std::min<int64_t>(lo[t.it.b], t.it.kv_begin);
      hi[t.it.b] = std::max<int64_t>(hi[t.it.b], t.it.kv_end);
    }
    int64_t keys = 0;
    for (int32_t b = 0; b < batch; ++b)
      if (hi[b] > lo[b]) keys += hi[b] - lo[b];
    if (keys * hkv * per_key > kLastLevelCacheBytes) {
      std::vector<int32_t> rank(batch, -1);
      int32_t next = 0;
      for (const Tmp& t : items)
        if (rank[t.it.b] < 0) rank[t.it.b] = next++;
      std::stable_sort(items.begin(), items.end(),
                       [&](const Tmp& a, const Tmp& b) { return rank[a.it.b] < rank[b.it.b]; });
    }
  }
  plan_header(plan, 2, params, cache, batch);
  plan->num_items = (int32_t)items.size();
  plan->num_merges = (int32_t)merges.size();
  plan->num_slots = (int32_t)num_slots;
  plan->chunk_blocks = (int32_t)chunk;
  plan->tile_rows = kPrefillTileRows;
  // Wave-stages of waves left without rows (a tile of rows r holds ceil(r / 16) busy
  // waves); from an eighth of all wave-stages on, the kernel form that lets such waves
  // skip the arithmetic is launched.
  int64_t wave_stages = 0, idle_stages = 0;
  for (const Tmp& t : items) {
    const int64_t s = stages_of(t.it);
    const int64_t busy = (t.it.row_end - t.it.row_begin + kPrefillWaveRows - 1) / kPrefillWaveRows;
    wave_stages += s * kPrefillWaves;
    idle_stages += s * (kPrefillWaves - busy);
  }
  plan->short_tiles = wave_stages > 0 && 8 * idle_stages >= wave_stages ? 1 : 0;
  plan->total_q = batch > 0 ? qo_indptr_host[batch] : 0;
  plan->max_kv_len = (int32_t)max_len;
  plan->items_offset = 0;
  plan->merges_offset = align_up((int64_t)items.size() * sizeof(PrefillItem), 16);
  plan->plan_bytes = align_up(plan->merges_offset + (int64_t)merges.size() * sizeof(PrefillMerge), 256);
  // Partials: o [slot][kv head][tile row][head_dim_vo] fp32; lse [slot][kv head][tile row]
  // x 2 fp32 (log2 domain: over the bf16-rounded weights, then over the fp32 weights).
  plan->partial_o_offset = plan->plan_bytes;
  const int64_t part_rows = num_slots * hkv * kPrefillTileRows;
  plan->partial_lse_offset = align_up(plan->partial_o_offset + part_rows * cache->head_dim_vo * 4, 256);
  plan->workspace_bytes = align_up(plan->partial_lse_offset + part_rows * 2 * 4, 256);
  plan->staged_pages = (int32_t)staged_pages;
  plan->staged_offset = 0;
  if (staged_pages > 0) {
    plan->staged_offset = plan->workspace_bytes;
    const int64_t rows = staged_pages * hkv * cache->page_size;
    plan->workspace_bytes = align_up(
        plan->staged_offset + rows * (cache->head_dim_qk + cache->head_dim_vo) * 2 + staged_pages * 4, 256);
  }
  if (!plan_buf_host) return PA_OK;
  if ((int64_t)plan_buf_bytes < plan->plan_bytes)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "plan buffer has %zu bytes, plan needs %lld",
                plan_buf_bytes, (long long)plan->plan_bytes);
  char* buf = (char*)plan_buf_host;
  memset(buf, 0, (size_t)plan->plan_bytes);
  PrefillItem* out = (PrefillItem*)(buf + plan->items_offset);
  for (size_t i = 0; i < items.size(); ++i) out[i] = items[i].it;
  if (!merges.empty())
    memcpy(buf + plan->merges_offset, merges.data(), merges.size() * sizeof(PrefillMerge));
  return PA_OK;
}

}  // extern "C"
