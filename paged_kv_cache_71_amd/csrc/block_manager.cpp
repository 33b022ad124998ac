// block_manager.cpp -- host-side block manager: free list, per-sequence block
// tables, reference counts and copy-on-write decisions.  CPU only; it builds
// the tables, slots and CoW pairs the kernels consume.
//
//  * A free list hands out blocks from its front in a caller-chosen order and
//    takes freed blocks back at its end; any free block will do (S06
//    PagedAttention chapter, "block manager" listing; kwkr.cn PagedAttention
//    post, KV-cache manager code).
//  * A sequence of n tokens holds ceil(n / B) blocks; a new block is taken only
//    when the last one is full, so waste stays below one block (CS349D lecture 3
//    sec. 3.1; CMU 11-868 lecture 24 sec. 3.1).
//  * fork shares every block of the parent (refcount + 1).  Appending into a
//    shared, partly filled last block first replaces it with a fresh private
//    copy (copy-on-write); the last holder writes in place.  Freeing drops
//    refcounts and returns blocks that reach zero (CS349D lecture 3 secs.
//    4.1-4.2; CMU 11-868 lecture 24 sec. 4).
//  * Exhaustion returns PKV_ERR_OOM and changes nothing (S06 chapter: the
//    allocator fails and the scheduler preempts).
//  * Swapping (CS349D lecture 3 sec. 5.2; "LLM inference, part 3", ch. 14): a
//    preempted sequence's blocks are copied to CPU blocks from a second free
//    list and its GPU blocks released (a block other sequences still hold
//    stays with them); swapping in takes fresh GPU blocks for its CPU blocks.
//    The (source, destination) pairs go to pkv_swap_blocks.  The CPU pool is
//    never larger than the caller makes it, so swap space stays bounded.
#include <deque>
#include <string>
#include <vector>

#include "pkv.h"

namespace pkv {
pkv_status fail(pkv_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
}
using pkv::fail;

struct pkv_block_manager {
  int32_t num_blocks = 0;
  int32_t B = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> refcount;
  int32_t num_cpu_blocks = 0;
  std::deque<int32_t> cpu_free;
  std::vector<char> cpu_used;
  struct Seq {
    bool live = false;
    bool swapped = false;  // its blocks are in cpu_table, its table is empty
    int32_t len = 0;
    std::vector<int32_t> table;
    std::vector<int32_t> cpu_table;
  };
  std::vector<Seq> seqs;

  const Seq* get(int32_t id) const {
    if (id < 0 || id >= (int32_t)seqs.size() || !seqs[id].live) return nullptr;
    return &seqs[id];
  }
  Seq* get(int32_t id) { return const_cast<Seq*>(static_cast<const pkv_block_manager*>(this)->get(id)); }
  // a live sequence whose blocks are on the GPU
  const Seq* resident(int32_t id) const {
    const Seq* sq = get(id);
    return sq && !sq->swapped ? sq : nullptr;
  }
  Seq* resident(int32_t id) { return const_cast<Seq*>(static_cast<const pkv_block_manager*>(this)->resident(id)); }
  int32_t new_seq_id() {
    seqs.emplace_back();
    return (int32_t)seqs.size() - 1;
  }
  int32_t take() {  // caller checked non-empty
    const int32_t b = free_list.front();
    free_list.pop_front();
    refcount[b] = 1;
    return b;
  }
  void release(int32_t b) {
    if (--refcount[b] == 0) free_list.push_back(b);
  }
};

namespace {
int32_t blocks_for(int64_t n, int32_t B) { return (int32_t)((n + B - 1) / B); }
}  // namespace

extern "C" {

pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                         pkv_block_manager** out) {
  if (!out) return fail(PKV_ERR_INVALID_ARG, "bm_create: null output");
  *out = nullptr;
  if (num_blocks < 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID_ARG, "bm_create: num_blocks=%d block_size=%d", num_blocks,
                block_size);
  auto* bm = new pkv_block_manager;
  bm->num_blocks = num_blocks;
  bm->B = block_size;
  bm->refcount.assign(num_blocks, 0);
  std::vector<char> seen(num_blocks, 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    const int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[b]) {
      delete bm;
      return fail(PKV_ERR_INVALID_ARG, "bm_create: free_order is not a permutation (entry %d = %d)",
                  i, b);
    }
    seen[b] = 1;
    bm->free_list.push_back(b);
  }
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

pkv_status pkv_bm_add_seq(pkv_block_manager* bm, int32_t n_tokens, int32_t* seq_id) {
  if (!bm || !seq_id || n_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "bm_add_seq: bad argument");
  const int32_t need = blocks_for(n_tokens, bm->B);
  if ((size_t)need > bm->free_list.size())
    return fail(PKV_ERR_OOM, "bm_add_seq: OOM (%d blocks needed, %zu free)", need,
                bm->free_list.size());
  const int32_t id = bm->new_seq_id();
  auto& sq = bm->seqs[id];
  sq.live = true;
  sq.len = n_tokens;
  for (int32_t i = 0; i < need; ++i) sq.table.push_back(bm->take());
  *seq_id = id;
  return PKV_OK;
}

pkv_status pkv_bm_append_token(pkv_block_manager* bm, int32_t seq_id, int64_t* slot,
                               int32_t* cow_src, int32_t* cow_dst) {
  if (!bm || !slot) return fail(PKV_ERR_INVALID_ARG, "bm_append_token: bad argument");
  auto* sq = bm->resident(seq_id);
  if (!sq) return fail(PKV_ERR_INVALID_ARG, "bm_append_token: no resident sequence %d", seq_id);
  const int32_t B = bm->B;
  const int32_t pos = sq->len;  // position of the new token
  int32_t src = -1, dst = -1;
  if (pos % B == 0) {
    // last block full (or no block yet): a fresh block, nothing to copy
    if (bm->free_list.empty()) return fail(PKV_ERR_OOM, "bm_append_token: OOM");
    sq->table.push_back(bm->take());
  } else {
    const int32_t last = sq->table.back();
    if (bm->refcount[last] > 1) {
      // shared, partly filled: copy-on-write into a fresh private block
      if (bm->free_list.empty()) return fail(PKV_ERR_OOM, "bm_append_token: OOM (copy-on-write)");
      const int32_t fresh = bm->take();
      bm->refcount[last] -= 1;  // still > 0: another sequence holds it
      sq->table.back() = fresh;
      src = last;
      dst = fresh;
    }
  }
  sq->len = pos + 1;
  *slot = (int64_t)sq->table[pos / B] * B + pos % B;
  if (cow_src) *cow_src = src;
  if (cow_dst) *cow_dst = dst;
  return PKV_OK;
}

pkv_status pkv_bm_fork(pkv_block_manager* bm, int32_t parent, int32_t* child) {
  if (!bm || !child) return fail(PKV_ERR_INVALID_ARG, "bm_fork: bad argument");
  if (!bm->resident(parent)) return fail(PKV_ERR_INVALID_ARG, "bm_fork: no resident sequence %d", parent);
  const int32_t id = bm->new_seq_id();  // may reallocate seqs: look the parent up again
  auto& p = bm->seqs[parent];
  auto& c = bm->seqs[id];
  c.live = true;
  c.len = p.len;
  c.table = p.table;
  for (int32_t b : c.table) bm->refcount[b] += 1;
  *child = id;
  return PKV_OK;
}

pkv_status pkv_bm_free_seq(pkv_block_manager* bm, int32_t seq_id) {
  if (!bm) return fail(PKV_ERR_INVALID_ARG, "bm_free_seq: null manager");
  auto* sq = bm->get(seq_id);
  if (!sq) return fail(PKV_ERR_INVALID_ARG, "bm_free_seq: no sequence %d", seq_id);
  for (int32_t b : sq->table) bm->release(b);
  for (int32_t c : sq->cpu_table) {
    bm->cpu_used[c] = 0;
    bm->cpu_free.push_back(c);
  }
  sq->table.clear();
  sq->cpu_table.clear();
  sq->swapped = false;
  sq->live = false;
  sq->len = 0;
  return PKV_OK;
}

pkv_status pkv_bm_table(const pkv_block_manager* bm, int32_t seq_id, int32_t* out, int32_t cap,
                        int32_t* n) {
  if (!bm || !n || cap < 0 || (cap > 0 && !out))
    return fail(PKV_ERR_INVALID_ARG, "bm_table: bad argument");
  const auto* sq = bm->resident(seq_id);
  if (!sq) return fail(PKV_ERR_INVALID_ARG, "bm_table: no resident sequence %d", seq_id);
  *n = (int32_t)sq->table.size();
  if (*n > cap) return fail(PKV_ERR_INVALID_ARG, "bm_table: capacity %d < %d", cap, *n);
  for (int32_t i = 0; i < *n; ++i) out[i] = sq->table[i];
  return PKV_OK;
}

pkv_status pkv_bm_seq_len(const pkv_block_manager* bm, int32_t seq_id, int32_t* n_tokens) {
  if (!bm || !n_tokens) return fail(PKV_ERR_INVALID_ARG, "bm_seq_len: bad argument");
  const auto* sq = bm->get(seq_id);
  if (!sq) return fail(PKV_ERR_INVALID_ARG, "bm_seq_len: no sequence %d", seq_id);
  *n_tokens = sq->len;
  return PKV_OK;
}

pkv_status pkv_bm_slots(const pkv_block_manager* bm, int32_t seq_id, int32_t start, int32_t count,
                        int64_t* out) {
  if (!bm || count < 0 || start < 0 || (count > 0 && !out))
    return fail(PKV_ERR_INVALID_ARG, "bm_slots: bad argument");
  const auto* sq = bm->resident(seq_id);
  if (!sq) return fail(PKV_ERR_INVALID_ARG, "bm_slots: no resident sequence %d", seq_id);
  if ((int64_t)start + count > sq->len)
    return fail(PKV_ERR_INVALID_ARG, "bm_slots: positions %d..%d past length %d", start,
                start + count - 1, sq->len);
  for (int32_t i = 0; i < count; ++i) {
    const int32_t pos = start + i;
    out[i] = (int64_t)sq->table[pos / bm->B] * bm->B + pos % bm->B;
  }
  return PKV_OK;
}

pkv_status pkv_bm_refcount(const pkv_block_manager* bm, int32_t block, int32_t* refcount) {
  if (!bm || !refcount || block < 0 || block >= bm->num_blocks)
    return fail(PKV_ERR_INVALID_ARG, "bm_refcount: bad argument");
  *refcount = bm->refcount[block];
  return PKV_OK;
}

pkv_status pkv_bm_num_free(const pkv_block_manager* bm, int32_t* n) {
  if (!bm || !n) return fail(PKV_ERR_INVALID_ARG, "bm_num_free: bad argument");
  *n = (int32_t)bm->free_list.size();
  return PKV_OK;
}

pkv_status pkv_bm_check(const pkv_block_manager* bm) {
  if (!bm) return fail(PKV_ERR_INVALID_ARG, "bm_check: null manager");
  std::vector<int32_t> holders(bm->num_blocks, 0);
  for (size_t i = 0; i < bm->seqs.size(); ++i) {
    const auto& sq = bm->seqs[i];
    if (!sq.live) continue;
    if (sq.swapped) {
      if (!sq.table.empty() || (int32_t)sq.cpu_table.size() != blocks_for(sq.len, bm->B))
        return fail(PKV_ERR_INVALID_ARG, "bm_check: swapped sequence %zu holds %zu / %zu blocks", i,
                    sq.table.size(), sq.cpu_table.size());
      continue;
    }
    if (!sq.cpu_table.empty())
      return fail(PKV_ERR_INVALID_ARG, "bm_check: resident sequence %zu holds CPU blocks", i);
    if ((int32_t)sq.table.size() != blocks_for(sq.len, bm->B))
      return fail(PKV_ERR_INVALID_ARG, "bm_check: sequence %zu has %zu blocks for %d tokens", i,
                  sq.table.size(), sq.len);
    for (int32_t b : sq.table) {
      if (b < 0 || b >= bm->num_blocks)
        return fail(PKV_ERR_INVALID_ARG, "bm_check: sequence %zu holds bad block %d", i, b);
      holders[b] += 1;
    }
  }
  std::vector<char> in_free(bm->num_blocks, 0);
  for (int32_t b : bm->free_list) {
    if (in_free[b]) return fail(PKV_ERR_INVALID_ARG, "bm_check: block %d free twice", b);
    in_free[b] = 1;
  }
  for (int32_t b = 0; b < bm->num_blocks; ++b) {
    if (holders[b] != bm->refcount[b])
      return fail(PKV_ERR_INVALID_ARG, "bm_check: block %d refcount %d but %d holders", b,
                  bm->refcount[b], holders[b]);
    if ((holders[b] == 0) != (in_free[b] != 0))
      return fail(PKV_ERR_INVALID_ARG, "bm_check: block %d free=%d with %d holders", b,
                  (int)in_free[b], holders[b]);
  }
  // CPU blocks: each held by exactly one swapped sequence or free, never both
  std::vector<int32_t> cpu_holders(bm->num_cpu_blocks, 0);
  for (const auto& sq : bm->seqs)
    if (sq.live)
      for (int32_t c : sq.cpu_table) {
        if (c < 0 || c >= bm->num_cpu_blocks) return fail(PKV_ERR_INVALID_ARG, "bm_check: bad CPU block %d", c);
        cpu_holders[c] += 1;
      }
  std::vector<char> cpu_in_free(bm->num_cpu_blocks, 0);
  for (int32_t c : bm->cpu_free) {
    if (cpu_in_free[c]) return fail(PKV_ERR_INVALID_ARG, "bm_check: CPU block %d free twice", c);
    cpu_in_free[c] = 1;
  }
  for (int32_t c = 0; c < bm->num_cpu_blocks; ++c)
    if (cpu_holders[c] > 1 || (cpu_holders[c] == 0) != (cpu_in_free[c] != 0) ||
        (cpu_holders[c] == 1) != (bm->cpu_used[c] != 0))
      return fail(PKV_ERR_INVALID_ARG, "bm_check: CPU block %d has %d holders, free=%d", c,
                  cpu_holders[c], (int)cpu_in_free[c]);
  return PKV_OK;
}

pkv_status pkv_bm_set_cpu_blocks(pkv_block_manager* bm, int32_t num_cpu_blocks) {
  if (!bm || num_cpu_blocks < 0) return fail(PKV_ERR_INVALID_ARG, "bm_set_cpu_blocks: bad argument");
  for (const auto& sq : bm->seqs)
    if (sq.live && sq.swapped)
      return fail(PKV_ERR_INVALID_ARG, "bm_set_cpu_blocks: a sequence is swapped out");
  bm->num_cpu_blocks = num_cpu_blocks;
  bm->cpu_free.clear();
  for (int32_t c = 0; c < num_cpu_blocks; ++c) bm->cpu_free.push_back(c);
  bm->cpu_used.assign(num_cpu_blocks, 0);
  return PKV_OK;
}

pkv_status pkv_bm_num_free_cpu(const pkv_block_manager* bm, int32_t* n) {
  if (!bm || !n) return fail(PKV_ERR_INVALID_ARG, "bm_num_free_cpu: bad argument");
  *n = (int32_t)bm->cpu_free.size();
  return PKV_OK;
}

pkv_status pkv_bm_swap_out(pkv_block_manager* bm, int32_t seq_id, int64_t* pairs, int32_t cap,
                           int32_t* n) {
  if (!bm || !n || cap < 0 || (cap > 0 && !pairs))
    return fail(PKV_ERR_INVALID_ARG, "bm_swap_out: bad argument");
  auto* sq = bm->resident(seq_id);
  if (!sq) return fail(PKV_ERR_INVALID_ARG, "bm_swap_out: no resident sequence %d", seq_id);
  const int32_t nb = (int32_t)sq->table.size();
  if (nb > cap) return fail(PKV_ERR_INVALID_ARG, "bm_swap_out: capacity %d < %d", cap, nb);
  if ((size_t)nb > bm->cpu_free.size())
    return fail(PKV_ERR_OOM, "bm_swap_out: OOM (%d CPU blocks needed, %zu free)", nb,
                bm->cpu_free.size());
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t c = bm->cpu_free.front();
    bm->cpu_free.pop_front();
    bm->cpu_used[c] = 1;
    pairs[2 * i] = sq->table[i];
    pairs[2 * i + 1] = c;
    sq->cpu_table.push_back(c);
    bm->release(sq->table[i]);
  }
  sq->table.clear();
  sq->swapped = true;
  *n = nb;
  return PKV_OK;
}

pkv_status pkv_bm_swap_in(pkv_block_manager* bm, int32_t seq_id, int64_t* pairs, int32_t cap,
                          int32_t* n) {
  if (!bm || !n || cap < 0 || (cap > 0 && !pairs))
    return fail(PKV_ERR_INVALID_ARG, "bm_swap_in: bad argument");
  auto* sq = bm->get(seq_id);
  if (!sq || !sq->swapped) return fail(PKV_ERR_INVALID_ARG, "bm_swap_in: no swapped sequence %d", seq_id);
  const int32_t nb = (int32_t)sq->cpu_table.size();
  if (nb > cap) return fail(PKV_ERR_INVALID_ARG, "bm_swap_in: capacity %d < %d", cap, nb);
  if ((size_t)nb > bm->free_list.size())
    return fail(PKV_ERR_OOM, "bm_swap_in: OOM (%d blocks needed, %zu free)", nb,
                bm->free_list.size());
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t g = bm->take();
    const int32_t c = sq->cpu_table[i];
    pairs[2 * i] = c;
    pairs[2 * i + 1] = g;
    sq->table.push_back(g);
    bm->cpu_used[c] = 0;
    bm->cpu_free.push_back(c);
  }
  sq->cpu_table.clear();
  sq->swapped = false;
  *n = nb;
  return PKV_OK;
}

}  // extern "C"
