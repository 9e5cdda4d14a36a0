// Randomised exercise of the library's host code — block manager, step composer and scheduler —
// through its C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer by
// test_host_sanitizers.py (no GPU involved).  Besides the sanitizers' own checks it verifies, after
// every call:
//   * block manager: each block's reference count equals the number of live table rows that hold
//     it, the free count equals the number of blocks nobody holds, appended slots follow the rows,
//     a copy-on-write replaces exactly the shared last block, and every rejected call (no space, or
//     a bad argument) leaves the whole state buffer byte for byte unchanged;
//   * step composer: decode tokens first, then chunks in queue order, within the budget;
//   * scheduler: planned rows, contexts and chunks stay in range, the rows' blocks are live, every
//     request finishes, all blocks come back, and the recorded times are ordered.
// Usage: host_fuzz SEED [ROUNDS]; exit status 0 when every check held.  A watchdog ends the run
// (SIGALRM) if a call never returns, as a corrupted queue or table would make it.
#include <unistd.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "pagedkv.h"

#define CHECK(c)                                                                     \
  do {                                                                               \
    if (!(c)) {                                                                      \
      std::fprintf(stderr, "check failed at %s:%d: %s\n", __FILE__, __LINE__, #c);   \
      std::exit(1);                                                                  \
    }                                                                                \
  } while (0)

namespace {

constexpr int kB = 16;

int blocks(int64_t tokens) { return static_cast<int>((tokens + kB - 1) / kB); }

struct Seq {
  std::vector<int32_t> row;     // max_blocks entries
  std::vector<int32_t> tokens;  // the prompt's token ids
  int32_t ctx = 0;
};

struct Bm {
  std::vector<uint64_t> buf;  // 8-byte aligned state
  int32_t nblk = 0;
  void* st() { return buf.data(); }
  std::vector<uint64_t> snapshot() const { return buf; }
  bool same(const std::vector<uint64_t>& s) const { return s == buf; }
};

void check_bm(Bm& bm, const std::vector<Seq>& seqs) {
  std::vector<int32_t> held(bm.nblk, 0);
  for (const Seq& s : seqs) {
    const int nb = blocks(s.ctx);
    for (int j = 0; j < nb; ++j) {
      CHECK(s.row[j] >= 0 && s.row[j] < bm.nblk);
      ++held[s.row[j]];
    }
    for (int j = 0; j < nb; ++j)
      for (int k = j + 1; k < nb; ++k) CHECK(s.row[j] != s.row[k]);
  }
  int32_t nfree = 0;
  for (int32_t b = 0; b < bm.nblk; ++b) {
    CHECK(pkv_bm_refcount(bm.st(), b) == held[b]);
    nfree += held[b] == 0;
  }
  CHECK(pkv_bm_num_free(bm.st()) == nfree);
  CHECK(pkv_bm_refcount(bm.st(), -1) == -1 && pkv_bm_refcount(bm.st(), bm.nblk) == -1);
}

void fuzz_block_manager(std::mt19937& rng, int rounds) {
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  Bm bm;
  bm.nblk = uni(1, 300);
  const int max_blocks = uni(1, 40);
  const size_t bytes = pkv_bm_state_bytes(bm.nblk);
  CHECK(bytes > 0);
  bm.buf.assign((bytes + 7) / 8, 0);
  std::vector<int32_t> order(bm.nblk);
  for (int i = 0; i < bm.nblk; ++i) order[i] = i;
  std::shuffle(order.begin(), order.end(), rng);
  const bool use_order = uni(0, 1);
  CHECK(pkv_bm_init(bm.st(), bytes, bm.nblk, kB, use_order ? order.data() : nullptr) == PKV_OK);
  // Bad initialisations leave nothing usable behind them, and report an error.
  {
    std::vector<uint64_t> other((bytes + 7) / 8, 0);
    std::vector<int32_t> dup(order);
    if (bm.nblk > 1) {
      dup[1] = dup[0];
      CHECK(pkv_bm_init(other.data(), bytes, bm.nblk, kB, dup.data()) == PKV_ERR_INVALID_ARG);
      CHECK(pkv_bm_num_free(other.data()) == -1);
    }
    CHECK(pkv_bm_init(other.data(), bytes - 8, bm.nblk, kB, nullptr) == PKV_ERR_WORKSPACE_TOO_SMALL);
    CHECK(pkv_bm_init(other.data(), bytes, bm.nblk, 8, nullptr) == PKV_ERR_UNSUPPORTED);
  }
  // A few base prompts, so that new prompts share prefixes with earlier ones.
  std::vector<std::vector<int32_t>> bases(4);
  for (auto& b : bases) {
    b.resize(max_blocks * kB);
    for (auto& t : b) t = uni(0, 5);  // a small alphabet: repeats inside one prompt happen too
  }
  std::vector<Seq> seqs;
  check_bm(bm, seqs);
  for (int it = 0; it < rounds; ++it) {
    const int op = uni(0, 9);
    if (op <= 2 || seqs.empty()) {  // add a sequence
      Seq s;
      s.row.assign(max_blocks, -7);
      const int n = uni(0, max_blocks * kB + 8);
      const auto& base = bases[uni(0, 3)];
      const int keep = uni(0, n);
      s.tokens.resize(n);
      for (int i = 0; i < n; ++i) s.tokens[i] = (i < keep && i < static_cast<int>(base.size())) ? base[i] : uni(0, 5);
      int32_t cached = -1;
      const auto before = bm.snapshot();
      const pkv_status r = pkv_bm_add_sequence(bm.st(), s.tokens.data(), n, s.row.data(), max_blocks, &cached);
      if (blocks(n) > max_blocks) {
        CHECK(r == PKV_ERR_INVALID_ARG && bm.same(before));
        continue;
      }
      if (r == PKV_ERR_NO_SPACE) {
        CHECK(bm.same(before));
        continue;
      }
      CHECK(r == PKV_OK);
      CHECK(cached >= 0 && cached % kB == 0 && cached <= (n / kB) * kB);
      for (int j = 0; j < cached / kB; ++j) CHECK(pkv_bm_block_hash(bm.st(), s.row[j]) != 0);
      for (int j = blocks(n); j < max_blocks; ++j) CHECK(s.row[j] == -7);  // nothing past the used entries
      s.ctx = n;
      seqs.push_back(std::move(s));
    } else if (op <= 5) {  // append
      Seq& s = seqs[uni(0, static_cast<int>(seqs.size()) - 1)];
      const int room = max_blocks * kB - s.ctx;
      const int num_new = uni(0, std::min(40, room + 3));
      std::vector<int32_t> slots(num_new + 1, -9), row_before(s.row);
      int32_t src = -9, dst = -9, ncopy = -9;
      const auto before = bm.snapshot();
      const pkv_status r =
          pkv_bm_append(bm.st(), s.row.data(), max_blocks, s.ctx, num_new, slots.data(), &src, &dst, &ncopy);
      if (num_new > room) {
        CHECK(r == PKV_ERR_INVALID_ARG && bm.same(before) && s.row == row_before);
        continue;
      }
      if (r == PKV_ERR_NO_SPACE) {
        CHECK(bm.same(before) && s.row == row_before);
        continue;
      }
      CHECK(r == PKV_OK);
      const int nb_old = blocks(s.ctx);
      if (ncopy == 1) {
        CHECK(num_new > 0 && s.ctx % kB != 0);
        CHECK(src == row_before[nb_old - 1] && dst == s.row[nb_old - 1] && src != dst);
        CHECK(pkv_bm_refcount(bm.st(), dst) == 1 && pkv_bm_refcount(bm.st(), src) >= 1);
      } else {
        CHECK(ncopy == 0);
        for (int j = 0; j < nb_old; ++j) CHECK(s.row[j] == row_before[j]);
      }
      for (int i = 0; i < num_new; ++i) {
        const int p = s.ctx + i;
        CHECK(slots[i] == s.row[p / kB] * kB + p % kB);
      }
      CHECK(slots[num_new] == -9);
      s.ctx += num_new;
    } else if (op == 6) {  // fork
      const Seq& p = seqs[uni(0, static_cast<int>(seqs.size()) - 1)];
      Seq c;
      c.row.assign(max_blocks, -7);
      c.tokens = p.tokens;
      c.ctx = p.ctx;
      CHECK(pkv_bm_fork(bm.st(), p.row.data(), p.ctx, c.row.data(), max_blocks) == PKV_OK);
      for (int j = 0; j < blocks(p.ctx); ++j) CHECK(c.row[j] == p.row[j]);
      seqs.push_back(std::move(c));
    } else if (op <= 8) {  // free
      const int k = uni(0, static_cast<int>(seqs.size()) - 1);
      CHECK(pkv_bm_free_sequence(bm.st(), seqs[k].row.data(), seqs[k].ctx) == PKV_OK);
      seqs.erase(seqs.begin() + k);
    } else {  // calls that must be rejected without touching the state
      const Seq& s = seqs[uni(0, static_cast<int>(seqs.size()) - 1)];
      const int nb = blocks(s.ctx);
      const auto before = bm.snapshot();
      std::vector<int32_t> row(s.row);
      if (nb >= 2) {  // a row that repeats a block
        row[nb - 1] = row[0];
        CHECK(pkv_bm_free_sequence(bm.st(), row.data(), s.ctx) == PKV_ERR_INVALID_ARG);
        CHECK(bm.same(before));
        row = s.row;
      }
      if (nb >= 1) {  // an id outside the pool
        row[uni(0, nb - 1)] = uni(0, 1) ? -1 : bm.nblk;
        int32_t sl[4], a, b, n;
        CHECK(pkv_bm_free_sequence(bm.st(), row.data(), s.ctx) == PKV_ERR_INVALID_ARG);
        CHECK(pkv_bm_append(bm.st(), row.data(), max_blocks, s.ctx, 1, sl, &a, &b, &n) == PKV_ERR_INVALID_ARG);
        std::vector<int32_t> child(max_blocks);
        CHECK(pkv_bm_fork(bm.st(), row.data(), s.ctx, child.data(), max_blocks) == PKV_ERR_INVALID_ARG);
        CHECK(bm.same(before));
      }
      int32_t cached, sl[2], a, b, n;
      CHECK(pkv_bm_append(bm.st(), nullptr, max_blocks, s.ctx, 1, sl, &a, &b, &n) == PKV_ERR_INVALID_ARG);
      CHECK(pkv_bm_append(bm.st(), row.data(), max_blocks, -1, 1, sl, &a, &b, &n) == PKV_ERR_INVALID_ARG);
      CHECK(pkv_bm_add_sequence(bm.st(), nullptr, 5, row.data(), max_blocks, &cached) == PKV_ERR_INVALID_ARG);
      CHECK(pkv_bm_add_sequence(bm.st(), s.tokens.data(), -1, row.data(), max_blocks, &cached) ==
            PKV_ERR_INVALID_ARG);
      CHECK(pkv_bm_free_sequence(nullptr, s.row.data(), s.ctx) == PKV_ERR_INVALID_ARG);
      CHECK(bm.same(before));
    }
    check_bm(bm, seqs);
  }
  for (const Seq& s : seqs) CHECK(pkv_bm_free_sequence(bm.st(), s.row.data(), s.ctx) == PKV_OK);
  seqs.clear();
  check_bm(bm, seqs);
  CHECK(pkv_bm_num_free(bm.st()) == bm.nblk);
}

void fuzz_compose(std::mt19937& rng, int rounds) {
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  for (int it = 0; it < rounds; ++it) {
    const int nd = uni(0, 300), np = uni(0, 12), budget = uni(1, 9000);
    const int cap = uni(0, 3) ? 0 : uni(1, 2048);
    std::vector<int32_t> rem(np), ch(np + 1, -5);
    for (auto& r : rem) r = uni(1, 5000);
    int32_t got = -1;
    CHECK(pkv_compose_step(nd, np ? rem.data() : nullptr, np, budget, cap, np ? ch.data() : nullptr, &got) ==
          PKV_OK);
    CHECK(got == std::min(nd, budget));
    int left = budget - got;
    for (int i = 0; i < np; ++i) {
      int c = std::min(rem[i], left);
      if (cap > 0) c = std::min(c, cap);
      CHECK(ch[i] == c);
      left -= c;
    }
    CHECK(left >= 0 && ch[np] == -5);
  }
  int32_t got, one = 0, ch;
  CHECK(pkv_compose_step(-1, nullptr, 0, 10, 0, nullptr, &got) == PKV_ERR_INVALID_ARG);
  CHECK(pkv_compose_step(1, &one, 1, 10, 0, &ch, &got) == PKV_ERR_INVALID_ARG);
  CHECK(pkv_compose_step(1, nullptr, 0, 0, 0, nullptr, &got) == PKV_ERR_INVALID_ARG);
}

void fuzz_scheduler(std::mt19937& rng, int mode) {
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  const int nblk = uni(40, 600), n = uni(1, 60), max_run = uni(1, 8), max_blocks = uni(8, 64);
  const int budget = uni(16, 512), max_chunk = uni(0, 2) ? 0 : uni(1, 128);
  std::vector<uint64_t> bmbuf((pkv_bm_state_bytes(nblk) + 7) / 8);
  CHECK(pkv_bm_init(bmbuf.data(), bmbuf.size() * 8, nblk, kB, nullptr) == PKV_OK);
  const int64_t itl_cap = 1 << 16;
  const size_t sb = pkv_sched_state_bytes(n, max_run, max_blocks, itl_cap);
  CHECK(sb > 0);
  std::vector<uint64_t> sbuf((sb + 7) / 8);
  void* st = sbuf.data();
  CHECK(pkv_sched_init(st, sb, mode, n, max_run, max_blocks, itl_cap, budget, max_chunk, bmbuf.data()) == PKV_OK);
  // Requests: a request fits the table row and, on its own, the pool.
  const int max_need = std::min(max_blocks, nblk);
  std::vector<int32_t> prompt(n), output(n);
  double t = 0.0;
  int64_t tokens_out = 0;
  for (int i = 0; i < n; ++i) {
    output[i] = uni(1, 40);
    prompt[i] = uni(1, std::max(1, max_need * kB - output[i] + 1));
    t += uni(0, 2) ? 0.0 : uni(1, 30) * 0.5;
    int32_t id = -1;
    CHECK(pkv_sched_add_request(st, prompt[i], output[i], t, &id) == PKV_OK && id == i);
    tokens_out += output[i];
  }
  {
    int32_t id;
    CHECK(pkv_sched_add_request(st, 5, 5, t - 1.0, &id) != PKV_OK);  // arrivals must not go back
    CHECK(pkv_sched_add_request(st, 0, 5, t, &id) == PKV_ERR_INVALID_ARG);
    CHECK(pkv_sched_add_request(st, 5, 5, NAN, &id) == PKV_ERR_INVALID_ARG);
  }
  std::vector<int32_t> dec_row(max_run), dec_ctx(max_run), ch_row(max_run), ch_off(max_run), ch_len(max_run);
  double now = 0.0;
  int steps = 0, done = 0;
  while (pkv_sched_num_done(st) < n) {
    int32_t nd = -1, nc = -1;
    double next = -2.0;
    CHECK(pkv_sched_plan(st, now, &nd, dec_row.data(), dec_ctx.data(), &nc, ch_row.data(), ch_off.data(),
                         ch_len.data(), &next) == PKV_OK);
    CHECK(nd >= 0 && nc >= 0 && nd + nc <= 2 * max_run);
    if (nd + nc == 0) {
      CHECK(next > now);
      now = next;
      continue;
    }
    if (mode == PKV_SCHED_NAIVE) CHECK(nd + nc == 1);
    int64_t step_tokens = nd;
    const int32_t* table = pkv_sched_table(st);
    auto row_live = [&](int32_t row, int64_t positions) {
      CHECK(row >= 0 && row < max_run);
      for (int j = 0; j < blocks(positions); ++j) {
        const int32_t b = table[static_cast<int64_t>(row) * max_blocks + j];
        CHECK(b >= 0 && b < nblk && pkv_bm_refcount(bmbuf.data(), b) >= 1);
      }
    };
    for (int i = 0; i < nd; ++i) {
      CHECK(dec_ctx[i] >= 2 && dec_ctx[i] <= max_blocks * kB);
      row_live(dec_row[i], dec_ctx[i]);
    }
    for (int i = 0; i < nc; ++i) {
      CHECK(ch_len[i] >= 1 && ch_off[i] >= 0 && ch_off[i] + ch_len[i] <= max_blocks * kB);
      if (max_chunk > 0 && mode == PKV_SCHED_CHUNKED) CHECK(ch_len[i] <= max_chunk);
      row_live(ch_row[i], static_cast<int64_t>(ch_off[i]) + ch_len[i]);
      step_tokens += ch_len[i];
    }
    if (mode == PKV_SCHED_CHUNKED) CHECK(step_tokens <= budget);
    now += 1.0 + static_cast<double>(step_tokens) / 64.0;
    CHECK(pkv_sched_complete(st, now) == PKV_OK);
    const int d = pkv_sched_num_done(st);
    CHECK(d >= done && d <= n);
    done = d;
    CHECK(++steps < 200000);
  }
  CHECK(pkv_bm_num_free(bmbuf.data()) == nblk);
  for (int i = 0; i < n; ++i) {
    double a, f, e;
    CHECK(pkv_sched_request_times(st, i, &a, &f, &e) == PKV_OK);
    CHECK(f >= a && e >= f);
  }
  std::vector<double> itl(itl_cap);
  const int64_t k = pkv_sched_itl(st, itl.data(), itl_cap);
  CHECK(k == tokens_out - n);
  for (int64_t i = 0; i < k; ++i) CHECK(itl[i] > 0.0);
}

}  // namespace

int main(int argc, char** argv) {
  const unsigned seed = argc > 1 ? static_cast<unsigned>(std::strtoul(argv[1], nullptr, 10)) : 1u;
  const int rounds = argc > 2 ? std::atoi(argv[2]) : 3000;
  alarm(120);
  std::mt19937 rng(seed);
  for (int r = 0; r < 8; ++r) fuzz_block_manager(rng, rounds);
  fuzz_compose(rng, rounds);
  for (int r = 0; r < 4; ++r)
    for (int mode = PKV_SCHED_NAIVE; mode <= PKV_SCHED_CHUNKED; ++mode) fuzz_scheduler(rng, mode);
  std::printf("host_fuzz seed %u: all checks held\n", seed);
  return 0;
}
