// Block manager for the paged KV pool (host code).
//
// What it does ("第2章:推理引擎核心技术", aiinfra.vidrealm.tech, §1.2, §1.5, §3.2; "C13 推理 · 第2课",
// section 改进二:PagedAttention, sharing paragraph): sequences get physical blocks through their
// block-table rows; blocks carry reference counts so that several sequences can point at the same
// block; a prompt's full blocks are found again by a chained hash of their token ids, and a hit
// shares the block; a shared, partly filled block is copied before a sequence writes into it.
//
// State: one caller-owned host buffer laid out as
//   Header | ref[N] | prev[N] | next[N] | hash[N] (u64) | table keys[T] (u64) | table values[T]
// with the free blocks in a doubly linked FIFO queue (prev/next, -1 = none) and an open-addressing
// hash table (linear probing, backward-shift deletion, key 0 = empty) from block hash to block.
// Every operation checks all its arguments and capacity before changing anything.
#include <cstddef>
#include <cstdint>
#include <cstring>

#include "pagedkv.h"

namespace {

constexpr uint32_t kMagic = 0x314d4b50u;  // "PKM1"
constexpr int32_t kB = 16;

struct Header {
  uint32_t magic;
  int32_t num_blocks;
  int32_t head, tail, nfree;
  int32_t table_size;  // power of two >= 2 * num_blocks
};

struct View {
  Header* h;
  int32_t* ref;
  int32_t* prev;
  int32_t* next;
  uint64_t* hash;
  uint64_t* keys;
  int32_t* vals;
};

size_t round8(size_t x) { return (x + 7) & ~static_cast<size_t>(7); }

int32_t table_size_for(int32_t n) {
  int32_t t = 16;
  while (t < 2 * n) t <<= 1;
  return t;
}

size_t bytes_for(int32_t n) {
  const size_t t = static_cast<size_t>(table_size_for(n));
  return round8(sizeof(Header)) + 3 * round8(4 * static_cast<size_t>(n)) + 8 * static_cast<size_t>(n) + 8 * t +
         round8(4 * t);
}

View view(void* state) {
  View v;
  char* p = static_cast<char*>(state);
  v.h = reinterpret_cast<Header*>(p);
  const int32_t n = v.h->num_blocks;
  const size_t t = static_cast<size_t>(v.h->table_size);
  p += round8(sizeof(Header));
  v.ref = reinterpret_cast<int32_t*>(p);
  p += round8(4 * static_cast<size_t>(n));
  v.prev = reinterpret_cast<int32_t*>(p);
  p += round8(4 * static_cast<size_t>(n));
  v.next = reinterpret_cast<int32_t*>(p);
  p += round8(4 * static_cast<size_t>(n));
  v.hash = reinterpret_cast<uint64_t*>(p);
  p += 8 * static_cast<size_t>(n);
  v.keys = reinterpret_cast<uint64_t*>(p);
  p += 8 * t;
  v.vals = reinterpret_cast<int32_t*>(p);
  return v;
}

bool valid(const void* state) {
  return state != nullptr && (reinterpret_cast<uintptr_t>(state) & 7) == 0 &&
         static_cast<const Header*>(state)->magic == kMagic;
}

// FNV-1a, 64-bit (Fowler, Noll and Vo): offset basis 14695981039346656037, prime 1099511628211.
uint64_t fnv1a(uint64_t h, const unsigned char* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 1099511628211ull;
  }
  return h;
}

// Hash of a full block: FNV-1a over the previous block's hash (8 bytes, little-endian) and the
// block's 16 token ids (4 bytes each, little-endian); 0 is reserved for "no hash".
uint64_t block_hash(uint64_t prev, const int32_t* tokens) {
  unsigned char buf[8 + 4 * kB];
  for (int i = 0; i < 8; ++i) buf[i] = static_cast<unsigned char>(prev >> (8 * i));
  for (int j = 0; j < kB; ++j) {
    const uint32_t t = static_cast<uint32_t>(tokens[j]);
    for (int i = 0; i < 4; ++i) buf[8 + 4 * j + i] = static_cast<unsigned char>(t >> (8 * i));
  }
  const uint64_t h = fnv1a(14695981039346656037ull, buf, sizeof(buf));
  return h ? h : 1;
}

// ---- hash table ---------------------------------------------------------------------------------
int32_t table_find(const View& v, uint64_t key) {
  const uint32_t mask = static_cast<uint32_t>(v.h->table_size - 1);
  for (uint32_t i = static_cast<uint32_t>(key) & mask;; i = (i + 1) & mask) {
    if (v.keys[i] == 0) return -1;
    if (v.keys[i] == key) return v.vals[i];
  }
}

void table_insert(View& v, uint64_t key, int32_t block) {
  const uint32_t mask = static_cast<uint32_t>(v.h->table_size - 1);
  for (uint32_t i = static_cast<uint32_t>(key) & mask;; i = (i + 1) & mask) {
    if (v.keys[i] == key) return;  // keep the block already registered under this hash
    if (v.keys[i] == 0) {
      v.keys[i] = key;
      v.vals[i] = block;
      return;
    }
  }
}

void table_erase(View& v, uint64_t key) {
  const uint32_t mask = static_cast<uint32_t>(v.h->table_size - 1);
  uint32_t i = static_cast<uint32_t>(key) & mask;
  while (v.keys[i] != key) {
    if (v.keys[i] == 0) return;
    i = (i + 1) & mask;
  }
  // Backward-shift deletion: move later entries of the probe run into the hole when their home
  // slot does not lie strictly between the hole and their position.
  for (uint32_t j = (i + 1) & mask;; j = (j + 1) & mask) {
    if (v.keys[j] == 0) break;
    const uint32_t home = static_cast<uint32_t>(v.keys[j]) & mask;
    const bool between = i <= j ? (i < home && home <= j) : (i < home || home <= j);
    if (!between) {
      v.keys[i] = v.keys[j];
      v.vals[i] = v.vals[j];
      i = j;
    }
  }
  v.keys[i] = 0;
  v.vals[i] = -1;
}

// ---- free queue ---------------------------------------------------------------------------------
void queue_push_back(View& v, int32_t b) {
  v.prev[b] = v.h->tail;
  v.next[b] = -1;
  if (v.h->tail >= 0) v.next[v.h->tail] = b; else v.h->head = b;
  v.h->tail = b;
  ++v.h->nfree;
}

void queue_remove(View& v, int32_t b) {
  if (v.prev[b] >= 0) v.next[v.prev[b]] = v.next[b]; else v.h->head = v.next[b];
  if (v.next[b] >= 0) v.prev[v.next[b]] = v.prev[b]; else v.h->tail = v.prev[b];
  v.prev[b] = v.next[b] = -1;
  --v.h->nfree;
}

// Takes the front of the queue for new content: its old hash registration (if any) is dropped.
int32_t take_fresh(View& v) {
  const int32_t b = v.h->head;
  queue_remove(v, b);
  if (v.hash[b] != 0) {
    if (table_find(v, v.hash[b]) == b) table_erase(v, v.hash[b]);
    v.hash[b] = 0;
  }
  v.ref[b] = 1;
  return b;
}

// A cached block found by its hash: shared (and out of the queue if it was waiting there).
void take_shared(View& v, int32_t b) {
  if (v.ref[b] == 0) queue_remove(v, b);
  ++v.ref[b];
}

bool table_row_ok(const View& v, const int32_t* row, int32_t nb) {
  for (int32_t j = 0; j < nb; ++j)
    if (row[j] < 0 || row[j] >= v.h->num_blocks || v.ref[row[j]] <= 0) return false;
  return true;
}

}  // namespace

extern "C" size_t pkv_bm_state_bytes(int32_t num_blocks) {
  if (num_blocks <= 0 || num_blocks > (1 << 28)) return 0;
  return bytes_for(num_blocks);
}

extern "C" pkv_status pkv_bm_init(void* state, size_t state_bytes, int32_t num_blocks, int32_t block_size,
                                  const int32_t* free_order) {
  if (block_size != kB) return PKV_ERR_UNSUPPORTED;
  if (!state || (reinterpret_cast<uintptr_t>(state) & 7) != 0 || num_blocks <= 0 || num_blocks > (1 << 28))
    return PKV_ERR_INVALID_ARG;
  if (state_bytes < bytes_for(num_blocks)) return PKV_ERR_WORKSPACE_TOO_SMALL;
  if (free_order)  // must be a permutation of 0 .. num_blocks-1; repeats are caught below
    for (int32_t i = 0; i < num_blocks; ++i)
      if (free_order[i] < 0 || free_order[i] >= num_blocks) return PKV_ERR_INVALID_ARG;
  std::memset(state, 0, bytes_for(num_blocks));
  Header* h = static_cast<Header*>(state);
  h->num_blocks = num_blocks;
  h->table_size = table_size_for(num_blocks);
  h->head = h->tail = -1;
  h->nfree = 0;
  View v = view(state);
  for (int32_t i = 0; i < h->table_size; ++i) v.vals[i] = -1;
  for (int32_t b = 0; b < num_blocks; ++b) v.prev[b] = v.next[b] = -2;  // -2: not yet queued
  for (int32_t i = 0; i < num_blocks; ++i) {
    const int32_t b = free_order ? free_order[i] : i;
    if (v.prev[b] != -2) {  // a repeated id: not a permutation
      std::memset(state, 0, sizeof(Header));
      return PKV_ERR_INVALID_ARG;
    }
    queue_push_back(v, b);
  }
  h->magic = kMagic;
  return PKV_OK;
}

extern "C" int32_t pkv_bm_num_free(const void* state) {
  if (!valid(state)) return -1;
  return static_cast<const Header*>(state)->nfree;
}

extern "C" int32_t pkv_bm_refcount(const void* state, int32_t block) {
  if (!valid(state)) return -1;
  View v = view(const_cast<void*>(state));
  if (block < 0 || block >= v.h->num_blocks) return -1;
  return v.ref[block];
}

extern "C" uint64_t pkv_bm_block_hash(const void* state, int32_t block) {
  if (!valid(state)) return 0;
  View v = view(const_cast<void*>(state));
  if (block < 0 || block >= v.h->num_blocks) return 0;
  return v.hash[block];
}

extern "C" pkv_status pkv_bm_add_sequence(void* state, const int32_t* tokens, int32_t num_tokens, int32_t* table_row,
                                          int32_t max_blocks, int32_t* cached_tokens) {
  if (!valid(state) || !table_row || !cached_tokens || num_tokens < 0 || max_blocks < 0 ||
      (num_tokens > 0 && !tokens))
    return PKV_ERR_INVALID_ARG;
  View v = view(state);
  const int32_t nb = (num_tokens + kB - 1) / kB;
  const int32_t nfull = num_tokens / kB;
  if (nb > max_blocks) return PKV_ERR_INVALID_ARG;
  // Longest cached prefix of full blocks.
  int32_t hits = 0;
  uint64_t h = 0;
  int32_t waiting = 0;  // hit blocks that sit in the free queue
  for (; hits < nfull; ++hits) {
    const uint64_t hj = block_hash(h, tokens + static_cast<size_t>(hits) * kB);
    const int32_t b = table_find(v, hj);
    if (b < 0) break;
    if (v.ref[b] == 0) ++waiting;
    h = hj;
  }
  if (v.h->nfree - waiting < nb - hits) return PKV_ERR_NO_SPACE;
  // Claim the hits, then allocate and register the rest.
  h = 0;
  for (int32_t j = 0; j < hits; ++j) {
    h = block_hash(h, tokens + static_cast<size_t>(j) * kB);
    const int32_t b = table_find(v, h);
    take_shared(v, b);
    table_row[j] = b;
  }
  for (int32_t j = hits; j < nb; ++j) {
    const int32_t b = take_fresh(v);
    table_row[j] = b;
    if (j < nfull) {
      h = block_hash(h, tokens + static_cast<size_t>(j) * kB);
      v.hash[b] = h;
      table_insert(v, h, b);
    }
  }
  *cached_tokens = hits * kB;
  return PKV_OK;
}

extern "C" pkv_status pkv_bm_append(void* state, int32_t* table_row, int32_t max_blocks, int32_t ctx, int32_t num_new,
                                    int32_t* slots, int32_t* copy_src, int32_t* copy_dst, int32_t* num_copies) {
  if (!valid(state) || !table_row || !num_copies || ctx < 0 || num_new < 0 || max_blocks < 0 ||
      (num_new > 0 && !slots))
    return PKV_ERR_INVALID_ARG;
  View v = view(state);
  const int32_t nb_old = (ctx + kB - 1) / kB;
  if (nb_old > max_blocks || !table_row_ok(v, table_row, nb_old)) return PKV_ERR_INVALID_ARG;
  *num_copies = 0;
  if (num_new == 0) return PKV_OK;
  const int64_t end = static_cast<int64_t>(ctx) + num_new;
  const int32_t nb_new = static_cast<int32_t>((end + kB - 1) / kB);
  if (nb_new > max_blocks) return PKV_ERR_INVALID_ARG;
  const bool cow = (ctx % kB) != 0 && v.ref[table_row[nb_old - 1]] > 1;
  if (cow && (!copy_src || !copy_dst)) return PKV_ERR_INVALID_ARG;
  if (v.h->nfree < (nb_new - nb_old) + (cow ? 1 : 0)) return PKV_ERR_NO_SPACE;
  if (cow) {
    const int32_t old = table_row[nb_old - 1];
    const int32_t fresh = take_fresh(v);
    --v.ref[old];  // stays >= 1: it was shared
    table_row[nb_old - 1] = fresh;
    copy_src[0] = old;
    copy_dst[0] = fresh;
    *num_copies = 1;
  }
  for (int32_t j = nb_old; j < nb_new; ++j) table_row[j] = take_fresh(v);
  for (int32_t i = 0; i < num_new; ++i) {
    const int32_t p = ctx + i;
    slots[i] = table_row[p / kB] * kB + p % kB;
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_bm_fork(void* state, const int32_t* parent_row, int32_t ctx, int32_t* child_row,
                                  int32_t max_blocks) {
  if (!valid(state) || !parent_row || !child_row || ctx < 0 || max_blocks < 0) return PKV_ERR_INVALID_ARG;
  View v = view(state);
  const int32_t nb = (ctx + kB - 1) / kB;
  if (nb > max_blocks || !table_row_ok(v, parent_row, nb)) return PKV_ERR_INVALID_ARG;
  for (int32_t j = 0; j < nb; ++j) {
    child_row[j] = parent_row[j];
    ++v.ref[parent_row[j]];
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_bm_free_sequence(void* state, const int32_t* table_row, int32_t ctx) {
  if (!valid(state) || !table_row || ctx < 0) return PKV_ERR_INVALID_ARG;
  View v = view(state);
  const int32_t nb = (ctx + kB - 1) / kB;
  if (!table_row_ok(v, table_row, nb)) return PKV_ERR_INVALID_ARG;
  // A row never repeats a block.  Blocks in use are out of the queue (next == -1), so next can
  // mark the blocks seen so far; the marks are cleared again before anything else changes.
  bool repeated = false;
  int32_t marked = 0;
  for (; marked < nb; ++marked) {
    int32_t& mark = v.next[table_row[marked]];
    if (mark == -3) {
      repeated = true;
      break;
    }
    mark = -3;
  }
  for (int32_t j = 0; j < marked; ++j) v.next[table_row[j]] = -1;
  if (repeated) return PKV_ERR_INVALID_ARG;
  for (int32_t j = 0; j < nb; ++j) {
    const int32_t b = table_row[j];
    if (--v.ref[b] == 0) queue_push_back(v, b);
  }
  return PKV_OK;
}
