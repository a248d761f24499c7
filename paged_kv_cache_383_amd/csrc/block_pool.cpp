// Host-side block pool: the scheduler's half of paged KV memory management.
//
// "PagedAttention" card (llm-engineer.pages.dev), "OS paging과 같은 발상" and
// "vLLM에서의 위치": the engine decides which physical KV blocks each request
// gets and appends a block to the request's block table when its cache grows;
// the GPU worker turns the tables into device tensors.  "vLLM KV cache and
// PagedAttention explained" (hrletsgo.me): Step 6 (ceil(n / 16) blocks at
// prefill, a new block at each block boundary during decode), Step 7 (a
// finished request's blocks return to the pool, immediately reusable), Step 9
// (blocks of a shared prefix carry a reference count; a write into a shared
// block first copies it into a new block that only the writer's table uses).
//
// Policy (the pages leave these open):
//   * token t of a sequence lives in logical block t / block_size;
//   * a block is copied only while another table still holds it (count > 1);
//     the last holder writes in place;
//   * allocation takes blocks from the front of an ordered free list, and the
//     blocks a free releases go back to the front in table order, so the next
//     request receives exactly the space just released;
//   * every operation is all-or-nothing: on PKV_ENOSPACE nothing changes.
#include <algorithm>
#include <deque>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"
#include "pkv_internal.h"

namespace {

pkv_status pool_fail(int code, const std::string& msg) { return pkv::set_error(code, msg); }

struct Sequence {
  std::vector<int32_t> table;
  int64_t tokens = 0;
};

}  // namespace

struct pkv_block_pool {
  int64_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;          // front = next block handed out
  std::vector<int32_t> refcount;          // tables holding each block
  std::unordered_map<int64_t, Sequence> seqs;

  int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }

  int32_t take() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    refcount[b] = 1;
    return b;
  }
};

extern "C" pkv_block_pool* pkv_pool_create(int64_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0) {
    pool_fail(PKV_EINVAL, "num_blocks must be in [1, 2^31) and block_size positive");
    return nullptr;
  }
  pkv_block_pool* p = new (std::nothrow) pkv_block_pool;
  if (!p) {
    pool_fail(PKV_EINVAL, "out of host memory");
    return nullptr;
  }
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->refcount.assign(size_t(num_blocks), 0);
  if (free_order) {
    std::vector<char> seen(size_t(num_blocks), 0);
    for (int64_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[size_t(b)]) {
        delete p;
        pool_fail(PKV_EINVAL, "free_order must list every block id in [0, num_blocks) exactly once");
        return nullptr;
      }
      seen[size_t(b)] = 1;
      p->free_list.push_back(b);
    }
  } else {
    for (int64_t b = 0; b < num_blocks; ++b) p->free_list.push_back(int32_t(b));
  }
  pkv::set_error(PKV_OK, "");
  return p;
}

extern "C" void pkv_pool_destroy(pkv_block_pool* p) { delete p; }

extern "C" pkv_status pkv_pool_allocate(pkv_block_pool* p, int64_t seq, int64_t num_tokens) {
  if (!p || num_tokens < 0) return pool_fail(PKV_EINVAL, "null pool or negative token count");
  if (p->seqs.count(seq)) return pool_fail(PKV_EINVAL, "sequence " + std::to_string(seq) + " already exists");
  const int64_t need = p->blocks_for(num_tokens);
  if (need > int64_t(p->free_list.size()))
    return pool_fail(PKV_ENOSPACE, std::to_string(need) + " blocks needed, " +
                                       std::to_string(p->free_list.size()) + " free");
  Sequence s;
  s.tokens = num_tokens;
  s.table.reserve(size_t(need));
  for (int64_t i = 0; i < need; ++i) s.table.push_back(p->take());
  p->seqs.emplace(seq, std::move(s));
  return pkv::set_error(PKV_OK, "");
}

extern "C" pkv_status pkv_pool_fork(pkv_block_pool* p, int64_t parent, int64_t child) {
  if (!p) return pool_fail(PKV_EINVAL, "null pool");
  auto it = p->seqs.find(parent);
  if (it == p->seqs.end()) return pool_fail(PKV_EINVAL, "unknown sequence " + std::to_string(parent));
  if (p->seqs.count(child)) return pool_fail(PKV_EINVAL, "sequence " + std::to_string(child) + " already exists");
  Sequence s = it->second;
  for (int32_t b : s.table) ++p->refcount[size_t(b)];
  p->seqs.emplace(child, std::move(s));
  return pkv::set_error(PKV_OK, "");
}

extern "C" pkv_status pkv_pool_append_slots(pkv_block_pool* p, int64_t seq, int64_t n, int64_t* slots_out,
                                     int64_t* copies_out, int64_t max_copies, int64_t* num_copies) {
  if (!p || n < 0 || (n > 0 && !slots_out) || !num_copies)
    return pool_fail(PKV_EINVAL, "null pool, output pointer or negative count");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return pool_fail(PKV_EINVAL, "unknown sequence " + std::to_string(seq));
  Sequence& s = it->second;
  const int64_t bs = p->block_size;
  // Blocks this call needs: one per boundary crossed, plus a private copy of
  // the partly filled last block when another table still holds it.
  int64_t need = p->blocks_for(s.tokens + n) - int64_t(s.table.size());
  const bool cow = n > 0 && s.tokens % bs != 0 && p->refcount[size_t(s.table.back())] > 1;
  if (cow) {
    ++need;
    if (max_copies < 1 || !copies_out) return pool_fail(PKV_EINVAL, "room for one block copy is needed");
  }
  if (need > int64_t(p->free_list.size()))
    return pool_fail(PKV_ENOSPACE, std::to_string(need) + " blocks needed, " +
                                       std::to_string(p->free_list.size()) + " free");
  *num_copies = 0;
  for (int64_t t = s.tokens; t < s.tokens + n; ++t) {
    const int64_t j = t / bs, off = t % bs;
    if (j == int64_t(s.table.size())) {
      s.table.push_back(p->take());
    } else if (p->refcount[size_t(s.table[size_t(j)])] > 1) {
      const int32_t src = s.table[size_t(j)];
      const int32_t dst = p->take();
      --p->refcount[size_t(src)];
      s.table[size_t(j)] = dst;
      copies_out[2 * *num_copies] = src;
      copies_out[2 * *num_copies + 1] = dst;
      ++*num_copies;
    }
    slots_out[t - s.tokens] = int64_t(s.table[size_t(j)]) * bs + off;
  }
  s.tokens += n;
  return pkv::set_error(PKV_OK, "");
}

extern "C" pkv_status pkv_pool_slots(const pkv_block_pool* p, int64_t seq, int64_t first, int64_t n, int64_t* slots_out) {
  if (!p || n < 0 || first < 0 || (n > 0 && !slots_out))
    return pool_fail(PKV_EINVAL, "null pool or output, or negative position or count");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return pool_fail(PKV_EINVAL, "unknown sequence " + std::to_string(seq));
  const Sequence& s = it->second;
  if (first + n > s.tokens)
    return pool_fail(PKV_EINVAL, "tokens [" + std::to_string(first) + ", " + std::to_string(first + n) +
                                     ") are not all held by sequence " + std::to_string(seq) + " (" +
                                     std::to_string(s.tokens) + " tokens)");
  const int64_t bs = p->block_size;
  for (int64_t t = first; t < first + n; ++t)
    slots_out[t - first] = int64_t(s.table[size_t(t / bs)]) * bs + t % bs;
  return pkv::set_error(PKV_OK, "");
}

extern "C" pkv_status pkv_pool_free(pkv_block_pool* p, int64_t seq) {
  if (!p) return pool_fail(PKV_EINVAL, "null pool");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return pool_fail(PKV_EINVAL, "unknown sequence " + std::to_string(seq));
  const std::vector<int32_t>& t = it->second.table;
  for (auto b = t.rbegin(); b != t.rend(); ++b)       // pushed in reverse: the front keeps table order
    if (--p->refcount[size_t(*b)] == 0) p->free_list.push_front(*b);
  p->seqs.erase(it);
  return pkv::set_error(PKV_OK, "");
}

extern "C" int64_t pkv_pool_num_free(const pkv_block_pool* p) { return p ? int64_t(p->free_list.size()) : -1; }

extern "C" int32_t pkv_pool_refcount(const pkv_block_pool* p, int64_t block) {
  if (!p || block < 0 || block >= p->num_blocks) return -1;
  return p->refcount[size_t(block)];
}

extern "C" int64_t pkv_pool_num_tokens(const pkv_block_pool* p, int64_t seq) {
  if (!p) return -1;
  auto it = p->seqs.find(seq);
  return it == p->seqs.end() ? -1 : it->second.tokens;
}

extern "C" int64_t pkv_pool_table(const pkv_block_pool* p, int64_t seq, int32_t* out, int64_t cap) {
  if (!p) return -1;
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return -1;
  const std::vector<int32_t>& t = it->second.table;
  for (int64_t i = 0; i < int64_t(t.size()) && i < cap; ++i) out[i] = t[size_t(i)];
  return int64_t(t.size());
}

extern "C" int64_t pkv_pool_free_list(const pkv_block_pool* p, int32_t* out, int64_t cap) {
  if (!p) return -1;
  int64_t i = 0;
  for (auto it = p->free_list.begin(); it != p->free_list.end() && i < cap; ++it) out[i++] = *it;
  return int64_t(p->free_list.size());
}

extern "C" pkv_status pkv_pool_usage(const pkv_block_pool* p, pkv_pool_usage_t* out) {
  if (!p || !out) return pool_fail(PKV_EINVAL, "null pool or output");
  // A used block stores the filled slots of its fullest holder, once, however
  // many tables share it.
  std::vector<int32_t> fill(size_t(p->num_blocks), -1);
  const int64_t bs = p->block_size;
  int64_t logical = 0;
  for (const auto& kv : p->seqs) {
    const Sequence& s = kv.second;
    logical += s.tokens;
    for (size_t j = 0; j < s.table.size(); ++j) {
      const int64_t f = std::min<int64_t>(bs, s.tokens - int64_t(j) * bs);
      int32_t& cur = fill[size_t(s.table[j])];
      cur = std::max<int32_t>(cur, int32_t(f));
    }
  }
  pkv_pool_usage_t u{};
  u.num_blocks = p->num_blocks;
  u.free_blocks = int64_t(p->free_list.size());
  u.sequences = int64_t(p->seqs.size());
  u.logical_tokens = logical;
  for (int64_t b = 0; b < p->num_blocks; ++b) {
    if (fill[size_t(b)] < 0) continue;
    ++u.used_blocks;
    u.stored_tokens += fill[size_t(b)];
    if (p->refcount[size_t(b)] > 1) ++u.shared_blocks;
  }
  u.allocated_slots = u.used_blocks * bs;
  *out = u;
  return pkv::set_error(PKV_OK, "");
}

extern "C" pkv_status pkv_pool_waste(const pkv_block_pool* p, int64_t max_model_len, int64_t bytes_per_token,
                              pkv_waste_t* out) {
  if (!p || !out || max_model_len < 0 || bytes_per_token < 0)
    return pool_fail(PKV_EINVAL, "null pool or output, or negative max_model_len / bytes_per_token");
  pkv_pool_usage_t u{};
  if (pkv_status rc = pkv_pool_usage(p, &u)) return rc;
  pkv_waste_t w{};
  w.empty_slots = u.allocated_slots - u.stored_tokens;
  w.paged_waste = u.allocated_slots ? double(w.empty_slots) / double(u.allocated_slots) : 0.0;
  w.static_slots = u.sequences * max_model_len;
  w.static_waste = w.static_slots ? 1.0 - double(u.logical_tokens) / double(w.static_slots) : 0.0;
  w.paged_bytes = u.allocated_slots * bytes_per_token;
  w.stored_bytes = u.stored_tokens * bytes_per_token;
  w.static_bytes = w.static_slots * bytes_per_token;
  *out = w;
  return pkv::set_error(PKV_OK, "");
}

extern "C" pkv_status pkv_account(const int64_t* lens, int32_t n, int32_t block_size, int32_t samples,
                           int64_t max_model_len, int64_t bytes_per_token, pkv_pool_usage_t* usage_out,
                           pkv_waste_t* waste_out) {
  if (n < 0 || (n > 0 && !lens) || block_size <= 0 || samples < 1 || !usage_out || !waste_out)
    return pool_fail(PKV_EINVAL, "bad lengths, block_size, samples or null output");
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (lens[i] < 0) return pool_fail(PKV_EINVAL, "negative request length");
    need += (lens[i] + block_size - 1) / block_size;
  }
  if (need > INT32_MAX) return pool_fail(PKV_EINVAL, "too many blocks");
  // Exactly the blocks the prompts need: forks share them and allocate nothing.
  pkv_block_pool* p = pkv_pool_create(std::max<int64_t>(need, 1), block_size, nullptr);
  if (!p) return pool_fail(PKV_EINVAL, "out of host memory");
  pkv_status rc = PKV_OK;
  for (int32_t i = 0; i < n && rc == PKV_OK; ++i) {
    rc = pkv_pool_allocate(p, int64_t(i) * samples, lens[i]);
    for (int32_t s = 1; s < samples && rc == PKV_OK; ++s)
      rc = pkv_pool_fork(p, int64_t(i) * samples, int64_t(i) * samples + s);
  }
  if (rc == PKV_OK) rc = pkv_pool_usage(p, usage_out);
  if (rc == PKV_OK) rc = pkv_pool_waste(p, max_model_len, bytes_per_token, waste_out);
  pkv_pool_destroy(p);
  return rc;
}

extern "C" pkv_status pkv_pool_build_tables(const pkv_block_pool* p, const int64_t* seqs, int32_t n, int32_t width,
                                     int32_t* tables_out, int32_t* lens_out) {
  if (!p || n < 0 || width <= 0 || (n > 0 && (!seqs || !tables_out || !lens_out)))
    return pool_fail(PKV_EINVAL, "null pool or output, or non-positive width");
  for (int32_t i = 0; i < n; ++i) {
    auto it = p->seqs.find(seqs[i]);
    if (it == p->seqs.end()) return pool_fail(PKV_EINVAL, "unknown sequence " + std::to_string(seqs[i]));
    const Sequence& s = it->second;
    if (int64_t(s.table.size()) > width)
      return pool_fail(PKV_EINVAL, "sequence " + std::to_string(seqs[i]) + " holds " +
                                       std::to_string(s.table.size()) + " blocks, wider than " +
                                       std::to_string(width));
    if (s.tokens > INT32_MAX) return pool_fail(PKV_EINVAL, "context length exceeds int32");
  }
  for (int32_t i = 0; i < n; ++i) {
    const Sequence& s = p->seqs.find(seqs[i])->second;
    int32_t* row = tables_out + int64_t(i) * width;
    for (int32_t j = 0; j < width; ++j) row[j] = j < int32_t(s.table.size()) ? s.table[size_t(j)] : -1;
    lens_out[i] = int32_t(s.tokens);
  }
  return pkv::set_error(PKV_OK, "");
}

// ---------------------------------------------------------------------------
// Batch: the rows of a decode batch and a mirror of the device block tables.
//
// A decode step's metadata lives on the GPU ([card] "vLLM에서의 위치": the
// worker keeps per-request block tables as device tensors).  Between two steps
// only a few entries change: each sequence grows by one token, which opens a
// new block every block_size steps, a copy-on-write replaces one entry, and a
// row whose request ended is reassigned.  The batch keeps a host mirror of the
// device tables, so each plan lists just the entries that differ; a kernel
// (paged_kv_prepare_step) applies them and derives the slot mapping on the
// device.
struct pkv_batch {
  pkv_block_pool* pool = nullptr;
  int32_t rows = 0, width = 0;
  std::vector<int64_t> seq;               // row -> sequence id, -1 = idle
  std::vector<int32_t> mirror;            // [rows, width]: what the device tables hold
  std::vector<int32_t> dirty_from;        // first column of the row that may differ (width = clean)
};

extern "C" pkv_batch* pkv_batch_create(pkv_block_pool* pool, int32_t rows, int32_t width) {
  if (!pool || rows <= 0 || width <= 0) {
    pool_fail(PKV_EINVAL, "null pool or non-positive rows / width");
    return nullptr;
  }
  pkv_batch* b = new (std::nothrow) pkv_batch;
  if (!b) {
    pool_fail(PKV_EINVAL, "out of host memory");
    return nullptr;
  }
  b->pool = pool;
  b->rows = rows;
  b->width = width;
  b->seq.assign(size_t(rows), -1);
  b->mirror.assign(size_t(rows) * size_t(width), -1);
  b->dirty_from.assign(size_t(rows), width);
  pkv::set_error(PKV_OK, "");
  return b;
}

extern "C" void pkv_batch_destroy(pkv_batch* b) { delete b; }

extern "C" pkv_status pkv_batch_set_row(pkv_batch* b, int32_t row, int64_t seq) {
  if (!b || row < 0 || row >= b->rows) return pool_fail(PKV_EINVAL, "null batch or row out of range");
  if (seq >= 0) {
    auto it = b->pool->seqs.find(seq);
    if (it == b->pool->seqs.end()) return pool_fail(PKV_EINVAL, "unknown sequence " + std::to_string(seq));
    if (int64_t(it->second.table.size()) > b->width)
      return pool_fail(PKV_EINVAL, "sequence " + std::to_string(seq) + " is wider than the batch tables");
  }
  b->seq[size_t(row)] = seq < 0 ? -1 : seq;
  b->dirty_from[size_t(row)] = 0;
  return pkv::set_error(PKV_OK, "");
}

extern "C" pkv_status pkv_batch_plan_step(pkv_batch* b, int32_t tokens_per_row, int32_t* updates_out, int64_t max_updates,
                                   int64_t* n_updates, int32_t* lens_out, int64_t* copies_out, int64_t max_copies,
                                   int64_t* n_copies) {
  if (!b || tokens_per_row < 0 || !n_updates || !lens_out || !n_copies || !updates_out ||
      (max_copies > 0 && !copies_out))
    return pool_fail(PKV_EINVAL, "null batch or output pointer, or negative token count");
  if (max_updates < int64_t(b->rows) * b->width)
    return pool_fail(PKV_EINVAL, "updates_out must hold rows * width = " +
                                     std::to_string(int64_t(b->rows) * b->width) + " entries");
  pkv_block_pool* p = b->pool;
  const int64_t bs = p->block_size;
  // Check first, so that a failure changes nothing: every active row's
  // sequence exists, stays within the table width, and the free list covers
  // the step's new blocks and copies.
  // A shared, partly filled last block X with reference count c that k rows
  // of the step append into is copied min(k, c - 1) times: each writer but
  // the last holder takes a private copy (pkv_pool_append_slots), and every
  // copy lowers X's count by one.
  int64_t need = 0, copies = 0;
  std::unordered_map<int32_t, int64_t> writers;        // shared last block -> rows appending into it
  for (int32_t r = 0; r < b->rows; ++r) {
    const int64_t s = b->seq[size_t(r)];
    if (s < 0) continue;
    auto it = p->seqs.find(s);
    if (it == p->seqs.end())
      return pool_fail(PKV_EINVAL, "row " + std::to_string(r) + " holds unknown sequence " + std::to_string(s));
    const Sequence& q = it->second;
    const int64_t nb = p->blocks_for(q.tokens + tokens_per_row);
    if (nb > b->width)
      return pool_fail(PKV_EINVAL, "sequence " + std::to_string(s) + " would outgrow the batch tables");
    need += nb - int64_t(q.table.size());
    if (tokens_per_row > 0 && q.tokens % bs != 0 && p->refcount[size_t(q.table.back())] > 1)
      ++writers[q.table.back()];
  }
  for (const auto& w : writers) copies += std::min<int64_t>(w.second, p->refcount[size_t(w.first)] - 1);
  need += copies;
  if (copies > max_copies) return pool_fail(PKV_EINVAL, "room for " + std::to_string(copies) + " copies is needed");
  if (need > int64_t(p->free_list.size()))
    return pool_fail(PKV_ENOSPACE, std::to_string(need) + " blocks needed, " +
                                       std::to_string(p->free_list.size()) + " free");
  // Count the updates before emitting any, for the same reason.
  *n_updates = 0;
  *n_copies = 0;
  int64_t slot_tmp[1];
  for (int32_t r = 0; r < b->rows; ++r) {
    const int64_t s = b->seq[size_t(r)];
    if (s < 0 || tokens_per_row == 0) continue;
    Sequence& q = p->seqs.find(s)->second;
    const int64_t first = q.tokens % bs != 0 ? int64_t(q.table.size()) - 1 : int64_t(q.table.size());
    for (int32_t t = 0; t < tokens_per_row; ++t) {
      int64_t nc = 0;
      pkv_pool_append_slots(p, s, 1, slot_tmp, copies_out + 2 * *n_copies, max_copies - *n_copies, &nc);
      *n_copies += nc;
    }
    int32_t& d = b->dirty_from[size_t(r)];
    d = std::min<int32_t>(d, int32_t(std::max<int64_t>(first, 0)));
  }
  for (int32_t r = 0; r < b->rows; ++r) {
    int32_t& d = b->dirty_from[size_t(r)];
    const int64_t s = b->seq[size_t(r)];
    const std::vector<int32_t>* t = s >= 0 ? &p->seqs.find(s)->second.table : nullptr;
    lens_out[r] = s >= 0 ? int32_t(p->seqs.find(s)->second.tokens) : 0;
    for (int32_t c = d; c < b->width; ++c) {
      const int32_t want = (t && c < int32_t(t->size())) ? (*t)[size_t(c)] : -1;
      int32_t& have = b->mirror[size_t(r) * b->width + c];
      if (have == want) continue;
      updates_out[3 * *n_updates] = r;
      updates_out[3 * *n_updates + 1] = c;
      updates_out[3 * *n_updates + 2] = want;
      ++*n_updates;
      have = want;
    }
    d = b->width;
  }
  return pkv::set_error(PKV_OK, "");
}
