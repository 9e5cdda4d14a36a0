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

// ---------------------------------------------------------------------------------------------
// Iteration-level scheduler over synthetic requests ("Phase 17 · 04 — vLLM serving internals",
// scheduler-loop section and its four modes; "第2章:推理引擎核心技术" §2.3).  Each step: release the
// finished requests and their blocks, admit waiting requests (queue order, only those that have
// arrived, while a running slot and enough KV blocks are free), then give every running request
// its work for the step: a whole-prompt prefill or a prompt chunk, or one decode token.  The
// caller runs the attention for the plan, then reports the step's end time; the scheduler records
// the first token (end of the step that finishes the prompt) and every later token.
// ---------------------------------------------------------------------------------------------

#include <cmath>
#include <cstring>

namespace {

constexpr uint32_t kSchedMagic = 0x31485350u;  // "PSH1"
enum : int32_t { kWaiting = 0, kPrefill = 1, kDecode = 2, kDone = 3, kReleased = 4 };

struct SchedHeader {
  uint32_t magic;
  int32_t mode, max_requests, max_running, max_blocks, token_budget, max_chunk;
  int32_t num_requests, next_waiting;  // requests are admitted in id order
  int32_t num_running, num_done;
  int64_t itl_capacity, itl_count;
  int64_t reserved_blocks;  // blocks running requests may still need
  void* bm;
  int32_t plan_decode, plan_chunks;
};

struct Req {
  int32_t prompt, output, state, row, prefilled, generated, admit_order, pad;
  double arrival, first, last, finish;
};

struct Sched {
  SchedHeader* h;
  Req* req;          // [max_requests]
  int32_t* running;  // [max_running] request ids in admission order
  int32_t* row_used; // [max_running]
  int32_t* table;    // [max_running][max_blocks]
  int32_t* plan;     // [3 * max_running]: decode ids, then (chunk id, chunk len) pairs
  int32_t* tokens;   // [16 * max_blocks]: synthetic prompt token ids handed to the block manager
  double* itl;       // [itl_capacity]
};

size_t r8(size_t x) { return (x + 7) & ~static_cast<size_t>(7); }

size_t sched_bytes(int32_t mr, int32_t mrun, int32_t mb, int64_t itl) {
  return r8(sizeof(SchedHeader)) + r8(sizeof(Req) * static_cast<size_t>(mr)) + r8(4 * static_cast<size_t>(mrun)) * 2 +
         r8(4 * static_cast<size_t>(mrun) * mb) + r8(12 * static_cast<size_t>(mrun)) + r8(64 * static_cast<size_t>(mb)) +
         8 * static_cast<size_t>(itl);
}

Sched sview(void* state) {
  Sched s;
  char* p = static_cast<char*>(state);
  s.h = reinterpret_cast<SchedHeader*>(p);
  p += r8(sizeof(SchedHeader));
  s.req = reinterpret_cast<Req*>(p);
  p += r8(sizeof(Req) * static_cast<size_t>(s.h->max_requests));
  s.running = reinterpret_cast<int32_t*>(p);
  p += r8(4 * static_cast<size_t>(s.h->max_running));
  s.row_used = reinterpret_cast<int32_t*>(p);
  p += r8(4 * static_cast<size_t>(s.h->max_running));
  s.table = reinterpret_cast<int32_t*>(p);
  p += r8(4 * static_cast<size_t>(s.h->max_running) * s.h->max_blocks);
  s.plan = reinterpret_cast<int32_t*>(p);
  p += r8(12 * static_cast<size_t>(s.h->max_running));
  s.tokens = reinterpret_cast<int32_t*>(p);
  p += r8(64 * static_cast<size_t>(s.h->max_blocks));
  s.itl = reinterpret_cast<double*>(p);
  return s;
}

bool sched_ok(const void* state) {
  return state && static_cast<const SchedHeader*>(state)->magic == kSchedMagic;
}

int32_t blocks_for(int64_t tokens) { return static_cast<int32_t>((tokens + 15) / 16); }
// Positions a request ever writes: its prompt and every generated token but the last.
int32_t need_blocks(const Req& r) { return blocks_for(static_cast<int64_t>(r.prompt) + r.output - 1); }
int32_t written(const Req& r) { return r.prompt + (r.generated > 0 ? r.generated - 1 : 0); }

void release(Sched& s, int32_t id) {
  Req& r = s.req[id];
  pkv_bm_free_sequence(s.h->bm, s.table + static_cast<int64_t>(r.row) * s.h->max_blocks, written(r));
  s.h->reserved_blocks -= need_blocks(r) - blocks_for(written(r));
  s.row_used[r.row] = 0;
  r.state = kReleased;
  int32_t k = 0;
  for (int32_t i = 0; i < s.h->num_running; ++i)
    if (s.running[i] != id) s.running[k++] = s.running[i];
  s.h->num_running = k;
}

}  // namespace

extern "C" size_t pkv_sched_state_bytes(int32_t max_requests, int32_t max_running, int32_t max_blocks,
                                        int64_t max_itl_samples) {
  if (max_requests <= 0 || max_running <= 0 || max_blocks <= 0 || max_itl_samples < 0) return 0;
  return sched_bytes(max_requests, max_running, max_blocks, max_itl_samples);
}

extern "C" pkv_status pkv_sched_init(void* state, size_t state_bytes, int32_t mode, int32_t max_requests,
                                     int32_t max_running, int32_t max_blocks, int64_t max_itl_samples,
                                     int32_t token_budget, int32_t max_chunk, void* bm_state) {
  if (!state || !bm_state || mode < PKV_SCHED_NAIVE || mode > PKV_SCHED_CHUNKED || max_requests <= 0 ||
      max_running <= 0 || max_blocks <= 0 || max_itl_samples < 0 || (mode == PKV_SCHED_CHUNKED && token_budget <= 0))
    return PKV_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(state) % 8 != 0) return PKV_ERR_INVALID_ARG;
  if (state_bytes < sched_bytes(max_requests, max_running, max_blocks, max_itl_samples))
    return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (pkv_bm_num_free(bm_state) < 0) return PKV_ERR_INVALID_ARG;
  std::memset(state, 0, sched_bytes(max_requests, max_running, max_blocks, max_itl_samples));
  SchedHeader* h = static_cast<SchedHeader*>(state);
  h->magic = kSchedMagic;
  h->mode = mode;
  h->max_requests = max_requests;
  h->max_running = max_running;  // NAIVE runs one request at a time but keeps the same layout
  h->max_blocks = max_blocks;
  h->token_budget = token_budget;
  h->max_chunk = max_chunk;
  h->itl_capacity = max_itl_samples;
  h->bm = bm_state;
  return PKV_OK;
}

extern "C" pkv_status pkv_sched_add_request(void* state, int32_t prompt_len, int32_t output_len, double arrival,
                                            int32_t* id) {
  if (!sched_ok(state) || !id || prompt_len <= 0 || output_len <= 0 || !std::isfinite(arrival))
    return PKV_ERR_INVALID_ARG;
  Sched s = sview(state);
  if (s.h->num_requests >= s.h->max_requests) return PKV_ERR_NO_SPACE;
  if (blocks_for(static_cast<int64_t>(prompt_len) + output_len - 1) > s.h->max_blocks) return PKV_ERR_INVALID_ARG;
  if (s.h->num_requests > 0 && arrival < s.req[s.h->num_requests - 1].arrival) return PKV_ERR_INVALID_ARG;
  const int32_t i = s.h->num_requests++;
  Req& r = s.req[i];
  std::memset(&r, 0, sizeof(Req));
  r.prompt = prompt_len;
  r.output = output_len;
  r.state = kWaiting;
  r.row = -1;
  r.arrival = arrival;
  r.first = r.last = r.finish = -1.0;
  *id = i;
  return PKV_OK;
}

extern "C" pkv_status pkv_sched_plan(void* state, double now, int32_t* num_decode, int32_t* dec_row, int32_t* dec_ctx,
                                     int32_t* num_chunks, int32_t* chunk_row, int32_t* chunk_offset,
                                     int32_t* chunk_len, double* next_arrival) {
  if (!sched_ok(state) || !num_decode || !dec_row || !dec_ctx || !num_chunks || !chunk_row || !chunk_offset ||
      !chunk_len || !next_arrival || !std::isfinite(now))
    return PKV_ERR_INVALID_ARG;
  Sched s = sview(state);
  SchedHeader& h = *s.h;
  const int32_t cap = h.mode == PKV_SCHED_NAIVE ? 1 : h.max_running;
  // Admission: NAIVE and STATIC only start a new batch once the previous one is fully released.
  const bool may_admit = (h.mode == PKV_SCHED_NAIVE || h.mode == PKV_SCHED_STATIC) ? h.num_running == 0 : true;
  while (may_admit && h.num_running < cap && h.next_waiting < h.num_requests) {
    Req& r = s.req[h.next_waiting];
    if (r.arrival > now) break;
    const int32_t need = need_blocks(r);
    if (static_cast<int64_t>(pkv_bm_num_free(h.bm)) - h.reserved_blocks < need) break;  // FIFO: wait for room
    int32_t row = 0;
    while (s.row_used[row]) ++row;
    int32_t* trow = s.table + static_cast<int64_t>(row) * h.max_blocks;
    for (int32_t j = 0; j < h.max_blocks; ++j) trow[j] = -1;
    // Synthetic prompt token ids, unique per request, so no prefix is shared between requests.
    const int32_t id = h.next_waiting;
    const int32_t P = r.prompt;
    for (int32_t p = 0; p < P; ++p) s.tokens[p] = (id << 20) ^ p ^ 0x5bd1e995;
    int32_t cached = 0;
    const pkv_status st = pkv_bm_add_sequence(h.bm, s.tokens, P, trow, h.max_blocks, &cached);
    if (st != PKV_OK) return st;
    s.row_used[row] = 1;
    r.row = row;
    r.state = kPrefill;
    r.admit_order = id;
    h.reserved_blocks += need - blocks_for(P);
    s.running[h.num_running++] = id;
    ++h.next_waiting;
  }
  // Work of the step.
  int32_t nd = 0, nc = 0;
  int32_t* plan_dec = s.plan;
  int32_t* plan_chunk = s.plan + h.max_running;  // (id, len) pairs
  int32_t budget_left = h.token_budget;
  for (int32_t i = 0; i < h.num_running; ++i) {  // decode tokens first
    Req& r = s.req[s.running[i]];
    if (r.state != kDecode) continue;
    if (h.mode == PKV_SCHED_CHUNKED) {
      if (budget_left == 0) break;
      --budget_left;
    }
    // The newest token (position prompt + generated - 1) is written this step.
    const int32_t ctx = r.prompt + r.generated;
    int32_t* trow = s.table + static_cast<int64_t>(r.row) * h.max_blocks;
    const int32_t before = blocks_for(ctx - 1);
    int32_t slot, cs, cd, ncp;
    const pkv_status st = pkv_bm_append(h.bm, trow, h.max_blocks, ctx - 1, 1, &slot, &cs, &cd, &ncp);
    if (st != PKV_OK) return st;
    h.reserved_blocks -= blocks_for(ctx) - before;
    dec_row[nd] = r.row;
    dec_ctx[nd] = ctx;
    plan_dec[nd++] = s.running[i];
  }
  for (int32_t i = 0; i < h.num_running; ++i) {  // then prompts, in admission order
    Req& r = s.req[s.running[i]];
    if (r.state != kPrefill) continue;
    int32_t len = r.prompt - r.prefilled;
    if (h.mode == PKV_SCHED_CHUNKED) {
      if (budget_left == 0) break;
      len = len < budget_left ? len : budget_left;
      if (h.max_chunk > 0 && len > h.max_chunk) len = h.max_chunk;
      budget_left -= len;
    }
    chunk_row[nc] = r.row;
    chunk_offset[nc] = r.prefilled;
    chunk_len[nc] = len;
    plan_chunk[2 * nc] = s.running[i];
    plan_chunk[2 * nc + 1] = len;
    ++nc;
  }
  h.plan_decode = nd;
  h.plan_chunks = nc;
  *num_decode = nd;
  *num_chunks = nc;
  *next_arrival = h.next_waiting < h.num_requests ? s.req[h.next_waiting].arrival : -1.0;
  return PKV_OK;
}

extern "C" const int32_t* pkv_sched_table(const void* state) {
  if (!sched_ok(state)) return nullptr;
  Sched s = sview(const_cast<void*>(state));
  return s.table;
}

extern "C" pkv_status pkv_sched_complete(void* state, double now) {
  if (!sched_ok(state) || !std::isfinite(now)) return PKV_ERR_INVALID_ARG;
  Sched s = sview(state);
  SchedHeader& h = *s.h;
  auto token = [&](Req& r) {
    if (r.generated == 0) {
      r.first = now;
    } else if (h.itl_count < h.itl_capacity) {
      s.itl[h.itl_count++] = now - r.last;
    }
    r.last = now;
    ++r.generated;
    if (r.generated == r.output) {
      r.state = kDone;
      r.finish = now;
      ++h.num_done;
    }
  };
  for (int32_t k = 0; k < h.plan_decode; ++k) token(s.req[s.plan[k]]);
  const int32_t* pc = s.plan + h.max_running;
  for (int32_t k = 0; k < h.plan_chunks; ++k) {
    Req& r = s.req[pc[2 * k]];
    r.prefilled += pc[2 * k + 1];
    if (r.prefilled == r.prompt) {
      r.state = kDecode;
      token(r);  // the step that finishes the prompt produces the first token
    }
  }
  h.plan_decode = h.plan_chunks = 0;
  // Release: STATIC keeps a finished request's slot until its whole batch has finished.
  bool all_done = true;
  for (int32_t i = 0; i < h.num_running; ++i) all_done &= s.req[s.running[i]].state == kDone;
  if (h.mode != PKV_SCHED_STATIC || all_done) {
    for (int32_t i = h.num_running - 1; i >= 0; --i)
      if (s.req[s.running[i]].state == kDone) release(s, s.running[i]);
  }
  return PKV_OK;
}

extern "C" int32_t pkv_sched_num_done(const void* state) {
  return sched_ok(state) ? static_cast<const SchedHeader*>(state)->num_done : -1;
}

extern "C" pkv_status pkv_sched_request_times(const void* state, int32_t id, double* arrival, double* first_token,
                                              double* finish) {
  if (!sched_ok(state) || !arrival || !first_token || !finish) return PKV_ERR_INVALID_ARG;
  Sched s = sview(const_cast<void*>(state));
  if (id < 0 || id >= s.h->num_requests) return PKV_ERR_INVALID_ARG;
  *arrival = s.req[id].arrival;
  *first_token = s.req[id].first;
  *finish = s.req[id].finish;
  return PKV_OK;
}

extern "C" int64_t pkv_sched_itl(const void* state, double* out, int64_t capacity) {
  if (!sched_ok(state) || capacity < 0 || (capacity > 0 && !out)) return -1;
  Sched s = sview(const_cast<void*>(state));
  const int64_t n = s.h->itl_count < capacity ? s.h->itl_count : capacity;
  for (int64_t i = 0; i < n; ++i) out[i] = s.itl[i];
  return s.h->itl_count;
}
