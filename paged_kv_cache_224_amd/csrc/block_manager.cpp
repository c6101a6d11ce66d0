// block_manager.cpp -- host-side block manager for the paged KV pool, behind the C ABI in
// include/pagedkv.h.
//
// What it keeps is fixed by the pages ("vllm-project-vllm -- L2", section 9 "Memory
// Management"; section 8 on the block-table invariant; section 11 steps 2 and 5): a sequence
// owns a list of fixed-size physical blocks that grows one block at a time as tokens are
// appended, so at most block_size - 1 slots of a sequence are ever unused; blocks can be
// shared copy-on-write (a fork is a table-pointer update, not a data copy); every physical
// block is free, owned by one table entry, or shared with a reference count equal to the
// number of table entries that name it; blocks of a preempted sequence can be swapped to a
// host pool and back.
//
// Policies the pages leave open, chosen here and stated in the header: the lowest-numbered
// free block is allocated first (device and host pools alike); a shared last block is
// copied when a sequence appends into it; a swap-out copies every block of the sequence
// (shared ones too) and a swap-in allocates fresh device blocks.

#include <cstdint>
#include <map>
#include <new>
#include <set>
#include <vector>

#include "pagedkv.h"

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;   // device block ids (or host ids while swapped out)
    int64_t ntok = 0;
    bool swapped = false;
  };
  int num_blocks = 0, block_size = 0, num_host_blocks = 0;
  std::vector<int32_t> ref;        // references per device block
  std::vector<int32_t> href;       // references per host block (0 or 1)
  std::set<int32_t> free_dev, free_host;
  std::map<int64_t, Seq> seqs;

  int32_t take(std::set<int32_t>& pool) {
    const int32_t b = *pool.begin();
    pool.erase(pool.begin());
    return b;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) free_dev.insert(b);
  }
  static int64_t blocks_for(int64_t ntok, int bs) { return (ntok + bs - 1) / bs; }
};

namespace {

using BM = pkv_block_manager;

BM::Seq* find(BM* m, int64_t id) {
  auto it = m->seqs.find(id);
  return it == m->seqs.end() ? nullptr : &it->second;
}

}  // namespace

extern "C" {

pkv_block_manager* pkv_bm_create(int num_blocks, int block_size, int num_host_blocks) {
  if (num_blocks < 0 || num_host_blocks < 0 || block_size <= 0) return nullptr;
  BM* m = new (std::nothrow) BM;
  if (!m) return nullptr;
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->num_host_blocks = num_host_blocks;
  m->ref.assign((size_t)num_blocks, 0);
  m->href.assign((size_t)num_host_blocks, 0);
  for (int32_t b = 0; b < num_blocks; ++b) m->free_dev.insert(m->free_dev.end(), b);
  for (int32_t b = 0; b < num_host_blocks; ++b) m->free_host.insert(m->free_host.end(), b);
  return m;
}

void pkv_bm_destroy(pkv_block_manager* m) { delete m; }

int pkv_bm_num_free(const pkv_block_manager* m) { return m ? (int)m->free_dev.size() : PKV_ERR_NULL; }

int pkv_bm_num_free_host(const pkv_block_manager* m) { return m ? (int)m->free_host.size() : PKV_ERR_NULL; }

int pkv_bm_add(pkv_block_manager* m, int64_t seq_id, int64_t num_tokens) {
  if (!m) return PKV_ERR_NULL;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (m->seqs.count(seq_id)) return PKV_ERR_STATE;
  const int64_t need = BM::blocks_for(num_tokens, m->block_size);
  if (need > (int64_t)m->free_dev.size()) return PKV_ERR_NO_SPACE;
  BM::Seq s;
  s.ntok = num_tokens;
  for (int64_t i = 0; i < need; ++i) {
    const int32_t b = m->take(m->free_dev);
    m->ref[b] = 1;
    s.blocks.push_back(b);
  }
  m->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

int pkv_bm_append(pkv_block_manager* m, int64_t seq_id, int64_t* slot, int32_t* copy_src,
                  int32_t* copy_dst) {
  if (!m || !slot || !copy_src || !copy_dst) return PKV_ERR_NULL;
  BM::Seq* s = find(m, seq_id);
  if (!s) return PKV_ERR_NOT_FOUND;
  if (s->swapped) return PKV_ERR_STATE;
  const int bs = m->block_size;
  const int64_t pos = s->ntok;                       // position of the new token
  *copy_src = *copy_dst = -1;
  if (pos % bs == 0) {                               // the last block is full (or none yet)
    if (m->free_dev.empty()) return PKV_ERR_NO_SPACE;
    const int32_t b = m->take(m->free_dev);
    m->ref[b] = 1;
    s->blocks.push_back(b);
  } else {
    const int32_t last = s->blocks.back();
    if (m->ref[last] > 1) {                          // shared partial block: copy on write
      if (m->free_dev.empty()) return PKV_ERR_NO_SPACE;
      const int32_t b = m->take(m->free_dev);
      m->ref[b] = 1;
      m->ref[last] -= 1;                             // still referenced by the other owners
      s->blocks.back() = b;
      *copy_src = last;
      *copy_dst = b;
    }
  }
  s->ntok = pos + 1;
  *slot = (int64_t)s->blocks.back() * bs + pos % bs;
  return PKV_OK;
}

int pkv_bm_fork(pkv_block_manager* m, int64_t parent, int64_t child, int64_t num_tokens) {
  if (!m) return PKV_ERR_NULL;
  BM::Seq* p = find(m, parent);
  if (!p) return PKV_ERR_NOT_FOUND;
  if (p->swapped || m->seqs.count(child)) return PKV_ERR_STATE;
  const int64_t n = num_tokens < 0 ? p->ntok : num_tokens;
  if (n > p->ntok) return PKV_ERR_SHAPE;
  BM::Seq c;
  c.ntok = n;
  const int64_t nb = BM::blocks_for(n, m->block_size);
  for (int64_t i = 0; i < nb; ++i) {
    const int32_t b = p->blocks[(size_t)i];
    m->ref[b] += 1;
    c.blocks.push_back(b);
  }
  m->seqs.emplace(child, std::move(c));
  return PKV_OK;
}

int pkv_bm_free(pkv_block_manager* m, int64_t seq_id) {
  if (!m) return PKV_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_ERR_NOT_FOUND;
  for (int32_t b : it->second.blocks) {
    if (it->second.swapped) {
      m->href[b] = 0;
      m->free_host.insert(b);
    } else {
      m->release(b);
    }
  }
  m->seqs.erase(it);
  return PKV_OK;
}

int pkv_bm_swap_out(pkv_block_manager* m, int64_t seq_id, int32_t* dev_blocks, int32_t* host_blocks,
                    int capacity) {
  if (!m || !dev_blocks || !host_blocks) return PKV_ERR_NULL;
  BM::Seq* s = find(m, seq_id);
  if (!s) return PKV_ERR_NOT_FOUND;
  if (s->swapped) return PKV_ERR_STATE;
  const int n = (int)s->blocks.size();
  if (n > capacity) return PKV_ERR_SHAPE;
  if (n > (int)m->free_host.size()) return PKV_ERR_NO_SPACE;
  for (int i = 0; i < n; ++i) {
    const int32_t d = s->blocks[(size_t)i];
    const int32_t h = m->take(m->free_host);
    m->href[h] = 1;
    dev_blocks[i] = d;
    host_blocks[i] = h;
    s->blocks[(size_t)i] = h;
    m->release(d);
  }
  s->swapped = true;
  return n;
}

int pkv_bm_swap_in(pkv_block_manager* m, int64_t seq_id, int32_t* host_blocks, int32_t* dev_blocks,
                   int capacity) {
  if (!m || !dev_blocks || !host_blocks) return PKV_ERR_NULL;
  BM::Seq* s = find(m, seq_id);
  if (!s) return PKV_ERR_NOT_FOUND;
  if (!s->swapped) return PKV_ERR_STATE;
  const int n = (int)s->blocks.size();
  if (n > capacity) return PKV_ERR_SHAPE;
  if (n > (int)m->free_dev.size()) return PKV_ERR_NO_SPACE;
  for (int i = 0; i < n; ++i) {
    const int32_t h = s->blocks[(size_t)i];
    const int32_t d = m->take(m->free_dev);
    m->ref[d] = 1;
    host_blocks[i] = h;
    dev_blocks[i] = d;
    s->blocks[(size_t)i] = d;
    m->href[h] = 0;
    m->free_host.insert(h);
  }
  s->swapped = false;
  return n;
}

int pkv_bm_num_tokens(const pkv_block_manager* m, int64_t seq_id, int64_t* num_tokens) {
  if (!m || !num_tokens) return PKV_ERR_NULL;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_ERR_NOT_FOUND;
  *num_tokens = it->second.ntok;
  return PKV_OK;
}

int pkv_bm_table(const pkv_block_manager* m, const int64_t* seq_ids, int num_seqs, int32_t* block_tables,
                 int max_blocks, int32_t* context_lens) {
  if (!m || (num_seqs > 0 && (!seq_ids || !block_tables || !context_lens))) return PKV_ERR_NULL;
  if (num_seqs < 0 || max_blocks < 0) return PKV_ERR_SHAPE;
  for (int i = 0; i < num_seqs; ++i) {
    auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end()) return PKV_ERR_NOT_FOUND;
    const BM::Seq& s = it->second;
    if (s.swapped) return PKV_ERR_STATE;
    if ((int64_t)s.blocks.size() > max_blocks || s.ntok > INT32_MAX) return PKV_ERR_SHAPE;
    int32_t* row = block_tables + (size_t)i * max_blocks;
    for (int j = 0; j < max_blocks; ++j) row[j] = j < (int)s.blocks.size() ? s.blocks[(size_t)j] : 0;
    context_lens[i] = (int32_t)s.ntok;
  }
  return PKV_OK;
}

int pkv_bm_check(const pkv_block_manager* m) {
  if (!m) return PKV_ERR_NULL;
  std::vector<int32_t> cnt((size_t)m->num_blocks, 0), hcnt((size_t)m->num_host_blocks, 0);
  for (const auto& kv : m->seqs) {
    const BM::Seq& s = kv.second;
    // a sequence holds exactly ceil(ntok / block_size) blocks: < block_size unused slots
    if ((int64_t)s.blocks.size() != BM::blocks_for(s.ntok, m->block_size)) return PKV_ERR_CHECK;
    for (int32_t b : s.blocks) {
      if (s.swapped) {
        if (b < 0 || b >= m->num_host_blocks || ++hcnt[(size_t)b] > 1) return PKV_ERR_CHECK;
      } else {
        if (b < 0 || b >= m->num_blocks) return PKV_ERR_CHECK;
        ++cnt[(size_t)b];
      }
    }
  }
  for (int32_t b = 0; b < m->num_blocks; ++b) {
    const bool is_free = m->free_dev.count(b) != 0;
    if (cnt[(size_t)b] != m->ref[(size_t)b]) return PKV_ERR_CHECK;     // refcount = references
    if (is_free != (cnt[(size_t)b] == 0)) return PKV_ERR_CHECK;         // free iff unreferenced
  }
  for (int32_t b = 0; b < m->num_host_blocks; ++b) {
    const bool is_free = m->free_host.count(b) != 0;
    if (hcnt[(size_t)b] != m->href[(size_t)b] || is_free != (hcnt[(size_t)b] == 0)) return PKV_ERR_CHECK;
  }
  return PKV_OK;
}

}  // extern "C"
