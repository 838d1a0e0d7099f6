// allocator.cpp — the host block allocator: free stack, reference counts, fork
// and copy on write of a shared tail block.
//
// Method: "KV Cache: capacity, layout, lifecycle", "Lifecycle and ownership"
// (free / exclusive / shared-read-only blocks; refcount = number of sequences
// holding the block; a shared block is copied before it is written; a block
// enters the free list only after its last GPU access; every release happens
// once; the table and the committed length change together) and "Reference
// counting and tail-block COW" (fork shares every block; the next token of a
// sequence takes a fresh block at a block boundary and copies a shared, partly
// filled tail first).  "03 | PagedAttention and the KV-cache memory system", §5
// (free queue, reference counts, fork of shared prefixes).
#include <hip/hip_runtime_api.h>

#include <mutex>
#include <vector>

#include "pagedkv.h"

struct pkv_alloc {
  int32_t num_blocks = 0, block_size = 0;
  std::vector<int32_t> refcount;  // per block
  std::vector<int32_t> free_stack;  // back = the next block handed out
  struct Seq {
    std::vector<int32_t> table;
    int64_t length = 0;  // committed tokens
    bool live = false;
  };
  std::vector<Seq> seqs;
  // blocks released behind an event: they become free once the event completes
  struct Pending {
    hipEvent_t event;
    std::vector<int32_t> blocks;
  };
  std::vector<Pending> pending;
  std::mutex mu;

  // move the blocks of every completed event onto the free stack (oldest first)
  void reclaim() {
    size_t keep = 0;
    for (size_t i = 0; i < pending.size(); ++i) {
      if (hipEventQuery(pending[i].event) == hipSuccess) {
        for (int32_t b : pending[i].blocks) free_stack.push_back(b);
      } else {
        if (keep != i) pending[keep] = std::move(pending[i]);  // never onto itself
        ++keep;
      }
    }
    pending.resize(keep);
  }

  // a fresh block with refcount 1, or -1 when none is free
  int32_t take() {
    if (free_stack.empty() && !pending.empty()) reclaim();
    if (free_stack.empty()) return -1;
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    refcount[b] = 1;
    return b;
  }

  Seq* seq(int32_t id) {
    if (id < 0 || id >= (int32_t)seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
};

extern "C" {

int pkv_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                     int32_t num_free, pkv_alloc** out) {
  if (!out || num_blocks < 1 || block_size < 1) return PKV_EINVAL;
  *out = nullptr;
  pkv_alloc* a = new pkv_alloc();
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->refcount.assign(num_blocks, 0);
  if (free_order) {
    if (num_free < 0 || num_free > num_blocks) {
      delete a;
      return PKV_EINVAL;
    }
    std::vector<uint8_t> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_free; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return PKV_EINVAL;
      }
      seen[b] = 1;
      a->free_stack.push_back(b);
    }
  } else {
    for (int32_t b = num_blocks - 1; b >= 0; --b) a->free_stack.push_back(b);
  }
  *out = a;
  return PKV_OK;
}

void pkv_alloc_destroy(pkv_alloc* a) { delete a; }

int pkv_alloc_add_seq(pkv_alloc* a, int32_t* seq) {
  if (!a || !seq) return PKV_EINVAL;
  std::lock_guard<std::mutex> lock(a->mu);
  a->seqs.emplace_back();
  a->seqs.back().live = true;
  *seq = (int32_t)a->seqs.size() - 1;
  return PKV_OK;
}

int pkv_alloc_fork(pkv_alloc* a, int32_t parent, int32_t* child) {
  if (!a || !child) return PKV_EINVAL;
  std::lock_guard<std::mutex> lock(a->mu);
  const pkv_alloc::Seq* p = a->seq(parent);
  if (!p) return PKV_EINVAL;
  pkv_alloc::Seq c;
  c.table = p->table;
  c.length = p->length;
  c.live = true;
  for (int32_t b : c.table) ++a->refcount[b];
  a->seqs.push_back(std::move(c));
  *child = (int32_t)a->seqs.size() - 1;
  return PKV_OK;
}

int pkv_alloc_append(pkv_alloc* a, int32_t seq, int64_t* slot, int32_t* cow_src,
                     int32_t* cow_dst) {
  if (!a || !slot) return PKV_EINVAL;
  std::lock_guard<std::mutex> lock(a->mu);
  pkv_alloc::Seq* s = a->seq(seq);
  if (!s) return PKV_EINVAL;
  const int64_t lb = s->length / a->block_size;
  const int32_t off = (int32_t)(s->length % a->block_size);
  int32_t src = -1, dst = -1;
  if (off == 0) {  // the token opens a block
    const int32_t b = a->take();
    if (b < 0) return PKV_ENOBLOCKS;
    s->table.push_back(b);
  } else if (a->refcount[s->table[lb]] > 1) {  // shared, partly filled tail: copy first
    const int32_t b = a->take();
    if (b < 0) return PKV_ENOBLOCKS;
    src = s->table[lb];
    dst = b;
    --a->refcount[src];
    s->table[lb] = b;
  }
  ++s->length;
  *slot = (int64_t)s->table[lb] * a->block_size + off;
  if (cow_src) *cow_src = src;
  if (cow_dst) *cow_dst = dst;
  return PKV_OK;
}

int pkv_alloc_free_seq(pkv_alloc* a, int32_t seq, void* event) {
  if (!a) return PKV_EINVAL;
  std::lock_guard<std::mutex> lock(a->mu);
  pkv_alloc::Seq* s = a->seq(seq);
  if (!s) return PKV_EINVAL;  // unknown, or released already: a release happens once
  hipEvent_t ev = static_cast<hipEvent_t>(event);
  if (ev) {
    const hipError_t q = hipEventQuery(ev);
    if (q != hipSuccess && q != hipErrorNotReady) return PKV_EINVAL;
  }
  std::vector<int32_t> released;
  for (auto it = s->table.rbegin(); it != s->table.rend(); ++it)
    if (--a->refcount[*it] == 0) released.push_back(*it);
  // the sequence's first block ends on top of the stack: released in reverse
  // table order, it is the first to be handed out again
  if (ev && !released.empty())
    a->pending.push_back({ev, std::move(released)});
  else
    for (int32_t b : released) a->free_stack.push_back(b);
  s->table.clear();
  s->table.shrink_to_fit();
  s->length = 0;
  s->live = false;
  return PKV_OK;
}

int pkv_alloc_block_table(pkv_alloc* a, int32_t seq, int32_t* table, int32_t capacity,
                          int32_t* num_blocks, int64_t* length) {
  if (!a || capacity < 0) return PKV_EINVAL;
  std::lock_guard<std::mutex> lock(a->mu);
  const pkv_alloc::Seq* s = a->seq(seq);
  if (!s) return PKV_EINVAL;
  const int32_t n = (int32_t)s->table.size();
  if (num_blocks) *num_blocks = n;
  if (length) *length = s->length;
  if (table) {
    if (capacity < n) return PKV_ERANGE;
    for (int32_t i = 0; i < n; ++i) table[i] = s->table[i];
  }
  return PKV_OK;
}

int pkv_alloc_refcount(pkv_alloc* a, int32_t block, int32_t* refcount) {
  if (!a || !refcount) return PKV_EINVAL;
  std::lock_guard<std::mutex> lock(a->mu);
  if (block < 0 || block >= a->num_blocks) return PKV_ERANGE;
  *refcount = a->refcount[block];
  return PKV_OK;
}

int pkv_alloc_free_blocks(pkv_alloc* a, int32_t* free_order, int32_t capacity,
                          int32_t* num_free) {
  if (!a || capacity < 0) return PKV_EINVAL;
  std::lock_guard<std::mutex> lock(a->mu);
  if (!a->pending.empty()) a->reclaim();
  const int32_t n = (int32_t)a->free_stack.size();
  if (num_free) *num_free = n;
  if (free_order) {
    if (capacity < n) return PKV_ERANGE;
    for (int32_t i = 0; i < n; ++i) free_order[i] = a->free_stack[i];
  }
  return PKV_OK;
}

}  // extern "C"
