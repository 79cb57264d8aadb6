// Paged prefill for gfx950 (placeholder until the MFMA kernel lands).
#include <hip/hip_runtime.h>

#include "pa_device.hpp"
#include "pa_internal.hpp"

using namespace pa;

extern "C" pa_status pa_paged_prefill(const pa_plan* plan, const void* q, const int32_t* qo_indptr,
                                      const pa_kv_cache* cache, const pa_page_table* table,
                                      const pa_attn_params* params, void* out, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  (void)plan; (void)q; (void)qo_indptr; (void)cache; (void)table; (void)params; (void)out;
  (void)lse; (void)workspace; (void)workspace_bytes; (void)stream;
  return fail(PA_ERR_UNSUPPORTED, "paged prefill is not built yet");
}
