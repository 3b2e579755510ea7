// block_manager.cpp -- host-side owner of the block pool: which pool block
// holds which positions of which sequence.  It hands out the block tables
// and slot numbers that the append and attention kernels consume.
//
// Rules (KV-cache visualization page, "PagedAttention: the cache in blocks";
// jovanaeducation guide, "Paging"):
//   - blocks of block_size token slots come from one shared pool, and each
//     sequence lists its blocks in order in its block table;
//   - a sequence takes a new block only when its last block is full, so at
//     most one of its blocks is partly filled;
//   - a finished sequence gives its blocks back at once;
//   - sequences with a common prefix point at the same blocks for it, and a
//     shared block is copied only when one of its holders writes into it.
// A block is shared by reference count.  The writer of a block held more than
// once moves onto a fresh block and reports the (source, destination) pair,
// which the caller copies on the GPU (pa_copy_blocks) before the append.
//
// Cost: add, fork and free are O(blocks touched); an append is O(tokens +
// requests); taking or returning a block is O(1) (a stack of free ids).
#include <algorithm>
#include <vector>

#include "pagedattn.h"
#include "status.h"

using pa::fail;

struct pa_block_manager {
  struct Seq {
    std::vector<int32_t> table;
    int32_t length = 0;
    bool live = false;
  };

  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ref;        // holders per block; 0 = free
  std::vector<int32_t> free_ids;   // stack of free blocks
  std::vector<Seq> seqs;           // indexed by sequence id
  std::vector<int32_t> free_seq_ids;

  int32_t take() {
    const int32_t b = free_ids.back();
    free_ids.pop_back();
    ref[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--ref[b] == 0) free_ids.push_back(b);
  }
  bool live(int32_t id) const {
    return id >= 0 && id < (int32_t)seqs.size() && seqs[id].live;
  }
  int32_t new_seq() {
    int32_t id;
    if (!free_seq_ids.empty()) {
      id = free_seq_ids.back();
      free_seq_ids.pop_back();
    } else {
      id = (int32_t)seqs.size();
      seqs.emplace_back();
    }
    seqs[id].live = true;
    seqs[id].length = 0;
    seqs[id].table.clear();
    return id;
  }
  int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }
};

namespace {

bool supported_block(int32_t bs) { return bs == 4 || bs == 8 || bs == 16 || bs == 32; }

}  // namespace

extern "C" {

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, pa_block_manager** out) {
  if (!out) return fail(PA_ERR_INVALID_ARG, "NULL result pointer");
  *out = nullptr;
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks %d must be positive", num_blocks);
  if (!supported_block(block_size))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not supported (4, 8, 16 or 32)", block_size);
  if ((int64_t)num_blocks * block_size > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "pool of %d blocks x %d slots exceeds 2^31 slots", num_blocks,
                block_size);
  auto* bm = new (std::nothrow) pa_block_manager;
  if (!bm) return fail(PA_ERR_INVALID_ARG, "out of host memory");
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  bm->free_ids.resize(num_blocks);
  for (int32_t i = 0; i < num_blocks; ++i) bm->free_ids[i] = num_blocks - 1 - i;  // 0 first
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status pa_bm_add_sequence(pa_block_manager* bm, int32_t* seq) {
  if (!bm || !seq) return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  *seq = bm->new_seq();
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t prefix_tokens, int32_t* child) {
  if (!bm || !child) return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  if (!bm->live(parent)) return fail(PA_ERR_INVALID_ARG, "sequence %d is not live", parent);
  const int32_t plen = bm->seqs[parent].length;
  const int32_t n = prefix_tokens < 0 ? plen : prefix_tokens;
  if (n > plen)
    return fail(PA_ERR_INVALID_ARG, "prefix of %d tokens is longer than sequence %d (%d)", n,
                parent, plen);
  const int32_t id = bm->new_seq();  // may grow seqs: index, do not hold references
  const int64_t nb = bm->blocks_for(n);
  auto& ptab = bm->seqs[parent].table;
  auto& ctab = bm->seqs[id].table;
  ctab.assign(ptab.begin(), ptab.begin() + nb);
  for (int32_t b : ctab) ++bm->ref[b];
  bm->seqs[id].length = n;
  *child = id;
  return PA_OK;
}

pa_status pa_bm_free_sequence(pa_block_manager* bm, int32_t seq) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "NULL manager");
  if (!bm->live(seq)) return fail(PA_ERR_INVALID_ARG, "sequence %d is not live", seq);
  auto& s = bm->seqs[seq];
  for (int32_t b : s.table) bm->drop(b);
  s.table.clear();
  s.table.shrink_to_fit();
  s.length = 0;
  s.live = false;
  bm->free_seq_ids.push_back(seq);
  return PA_OK;
}

pa_status pa_bm_append(pa_block_manager* bm, const int32_t* seqs, const int32_t* num_tokens,
                       int32_t num_requests, int64_t* slots, int64_t max_slots, int32_t* copies,
                       int32_t max_copies, int32_t* num_copies) {
  if (!bm || !num_copies) return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  *num_copies = 0;
  if (num_requests < 0) return fail(PA_ERR_INVALID_ARG, "num_requests %d < 0", num_requests);
  if (num_requests == 0) return PA_OK;
  if (!seqs || !num_tokens) return fail(PA_ERR_INVALID_ARG, "NULL request arrays");
  // Every check first; nothing changes unless the whole append fits.
  const int32_t bs = bm->block_size;
  int64_t total = 0;
  for (int32_t r = 0; r < num_requests; ++r) {
    const int32_t id = seqs[r];
    if (!bm->live(id)) return fail(PA_ERR_INVALID_ARG, "request %d: sequence %d is not live", r, id);
    if (num_tokens[r] < 0)
      return fail(PA_ERR_INVALID_ARG, "request %d: %d tokens", r, num_tokens[r]);
    if ((int64_t)bm->seqs[id].length + num_tokens[r] > (int64_t)bm->num_blocks * bs)
      return fail(PA_ERR_OUT_OF_BLOCKS, "request %d: %lld tokens exceed the pool", r,
                  (long long)bm->seqs[id].length + num_tokens[r]);
    total += num_tokens[r];
  }
  {
    std::vector<int32_t> ids(seqs, seqs + num_requests);
    std::sort(ids.begin(), ids.end());
    if (std::adjacent_find(ids.begin(), ids.end()) != ids.end())
      return fail(PA_ERR_INVALID_ARG, "a sequence appears twice in one append");
  }
  // The exact number of fresh blocks, following the requests in order: once
  // one holder of a shared last block has copied it away, a later holder may
  // be its only one and writes in place.
  int64_t need = 0;
  int32_t ncopy = 0;
  std::vector<int32_t> lowered;  // provisional count drops, undone below
  for (int32_t r = 0; r < num_requests; ++r) {
    const auto& s = bm->seqs[seqs[r]];
    if (num_tokens[r] == 0) continue;
    need += bm->blocks_for((int64_t)s.length + num_tokens[r]) - bm->blocks_for(s.length);
    if (s.length % bs && bm->ref[s.table.back()] > 1) {
      ++need;
      ++ncopy;
      --bm->ref[s.table.back()];
      lowered.push_back(s.table.back());
    }
  }
  for (int32_t b : lowered) ++bm->ref[b];
  if (total > 0 && !slots) return fail(PA_ERR_INVALID_ARG, "NULL slots");
  if (total > max_slots)
    return fail(PA_ERR_INVALID_ARG, "slots buffer holds %lld, the append needs %lld",
                (long long)max_slots, (long long)total);
  if (ncopy > 0 && (!copies || ncopy > max_copies))
    return fail(PA_ERR_INVALID_ARG, "copies buffer holds %d pairs, the append needs %d",
                copies ? max_copies : 0, ncopy);
  if (need > (int64_t)bm->free_ids.size())
    return fail(PA_ERR_OUT_OF_BLOCKS, "the append needs %lld free blocks, %zu are free",
                (long long)need, bm->free_ids.size());

  int64_t t = 0;
  for (int32_t r = 0; r < num_requests; ++r) {
    auto& s = bm->seqs[seqs[r]];
    for (int32_t i = 0; i < num_tokens[r]; ++i) {
      const int32_t pos = s.length;
      if (pos % bs == 0) {
        s.table.push_back(bm->take());
      } else if (bm->ref[s.table.back()] > 1) {  // first write into a shared block
        const int32_t src = s.table.back();
        const int32_t dst = bm->take();
        copies[2 * *num_copies] = src;
        copies[2 * *num_copies + 1] = dst;
        ++*num_copies;
        bm->drop(src);
        s.table.back() = dst;
      }
      slots[t++] = (int64_t)s.table[pos / bs] * bs + pos % bs;
      ++s.length;
    }
  }
  return PA_OK;
}

pa_status pa_bm_block_tables(const pa_block_manager* bm, const int32_t* seqs, int32_t num_seqs,
                             int32_t max_blocks_per_seq, int32_t* block_tables,
                             int32_t* context_lens) {
  if (!bm) return fail(PA_ERR_INVALID_ARG, "NULL manager");
  if (num_seqs < 0 || max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "bad sizes");
  if (num_seqs == 0) return PA_OK;
  if (!seqs || !block_tables) return fail(PA_ERR_INVALID_ARG, "NULL pointer");
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (!bm->live(seqs[i])) return fail(PA_ERR_INVALID_ARG, "sequence %d is not live", seqs[i]);
    const auto& tab = bm->seqs[seqs[i]].table;
    if ((int64_t)tab.size() > max_blocks_per_seq)
      return fail(PA_ERR_INVALID_ARG, "sequence %d holds %zu blocks, the table row %d", seqs[i],
                  tab.size(), max_blocks_per_seq);
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const auto& s = bm->seqs[seqs[i]];
    int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
    std::copy(s.table.begin(), s.table.end(), row);
    std::fill(row + s.table.size(), row + max_blocks_per_seq, -1);
    if (context_lens) context_lens[i] = s.length;
  }
  return PA_OK;
}

int32_t pa_bm_num_free_blocks(const pa_block_manager* bm) {
  return bm ? (int32_t)bm->free_ids.size() : -1;
}

int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

int32_t pa_bm_sequence_length(const pa_block_manager* bm, int32_t seq) {
  if (!bm || !bm->live(seq)) return -1;
  return bm->seqs[seq].length;
}

}  // extern "C"
