// Step composition for mixed decode / chunked-prefill batches (host code).
//
// The rule ("Chunked Prefill", Ultralytics, token-budget section; "Phase 17 · 04 — vLLM serving
// internals", scheduler-loop section): every step has a token budget; each running sequence first
// gets one decode token, then the waiting prompts, in queue order, fill what is left with chunks; a
// prompt that does not fit goes on in the next step.
#include <cstdint>

#include "pagedkv.h"

extern "C" pkv_status pkv_compose_step(int32_t num_decode, const int32_t* prefill_remaining, int32_t num_prefill,
                                       int32_t token_budget, int32_t max_chunk, int32_t* chunk_len,
                                       int32_t* num_decode_scheduled) {
  if (num_decode < 0 || num_prefill < 0 || token_budget <= 0 || !num_decode_scheduled) return PKV_ERR_INVALID_ARG;
  if (num_prefill > 0 && (!prefill_remaining || !chunk_len)) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < num_prefill; ++i)
    if (prefill_remaining[i] <= 0) return PKV_ERR_INVALID_ARG;
  const int32_t dec = num_decode < token_budget ? num_decode : token_budget;
  int32_t left = token_budget - dec;
  for (int32_t i = 0; i < num_prefill; ++i) {
    int32_t c = prefill_remaining[i] < left ? prefill_remaining[i] : left;
    if (max_chunk > 0 && c > max_chunk) c = max_chunk;
    chunk_len[i] = c;
    left -= c;
  }
  *num_decode_scheduled = dec;
  return PKV_OK;
}
