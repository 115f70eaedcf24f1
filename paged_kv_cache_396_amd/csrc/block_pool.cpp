// Host-side KV block pool; the policy is described in block_pool.h.
#include "block_pool.h"

#include <string.h>

namespace pa {

namespace {
constexpr uint64_t kRoot = 0x243f6a8885a308d3ull;  // parent hash of a sequence's first block

uint64_t mix64(uint64_t x) {  // splitmix64 finaliser
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}
}  // namespace

BlockPool::BlockPool(int32_t num_blocks) : blocks_(num_blocks > 0 ? num_blocks : 0) {
  for (int32_t b = 1; b < num_blocks; ++b) queue_push_tail(b);
}

uint64_t BlockPool::chain_hash(uint64_t parent, const int32_t* tokens) {
  uint64_t h = mix64(parent);
  for (int i = 0; i < kTokens; ++i) h = mix64(h ^ (uint64_t)(uint32_t)tokens[i]);
  return h;
}

// Block holding exactly (parent, tokens), or -1.
int32_t BlockPool::lookup(uint64_t parent, const int32_t* tokens) const {
  auto it = index_.find(chain_hash(parent, tokens));
  if (it == index_.end()) return -1;
  const Block& k = blocks_[it->second];
  if (k.parent_hash != parent || memcmp(k.tokens, tokens, sizeof(k.tokens)) != 0) return -1;
  return it->second;
}

void BlockPool::queue_remove(int32_t b) {
  Block& k = blocks_[b];
  if (k.prev >= 0) blocks_[k.prev].next = k.next; else head_ = k.next;
  if (k.next >= 0) blocks_[k.next].prev = k.prev; else tail_ = k.prev;
  k.prev = k.next = -1;
  k.in_free = false;
  --num_free_;
}

void BlockPool::queue_push_tail(int32_t b) {
  Block& k = blocks_[b];
  k.prev = tail_;
  k.next = -1;
  if (tail_ >= 0) blocks_[tail_].next = b; else head_ = b;
  tail_ = b;
  k.in_free = true;
  ++num_free_;
}

// Least recently used free block, with its old index entry dropped.
int32_t BlockPool::take_head() {
  const int32_t b = head_;
  queue_remove(b);
  Block& k = blocks_[b];
  if (k.keyed) {
    index_.erase(k.hash);
    k.keyed = false;
  }
  k.ref = 1;
  return b;
}

int BlockPool::add_request(int64_t req, const int32_t* prompt, int32_t n, int32_t* num_cached) {
  if (reqs_.count(req)) return -2;
  Request r;
  uint64_t parent = kRoot;
  const int32_t lookups = n > 0 ? (n - 1) / kTokens : 0;
  for (int32_t j = 0; j < lookups; ++j) {
    const int32_t b = lookup(parent, prompt + j * kTokens);
    if (b < 0) break;
    Block& k = blocks_[b];
    if (k.ref == 0) queue_remove(b);
    ++k.ref;
    r.blocks.push_back(b);
    parent = k.hash;
  }
  r.tokens.assign(prompt, prompt + r.blocks.size() * kTokens);
  *num_cached = (int32_t)r.tokens.size();
  reqs_.emplace(req, std::move(r));
  return 0;
}

int BlockPool::allocate_slots(int64_t req, const int32_t* tokens, int32_t n, int64_t* slots,
                              int32_t* copy, int32_t* num_copies) {
  auto it = reqs_.find(req);
  if (it == reqs_.end()) return -1;
  Request& r = it->second;
  const int64_t T = (int64_t)r.tokens.size();
  const bool cow = T % kTokens != 0 && blocks_[r.blocks.back()].ref > 1;
  const int64_t need = (T + n + kTokens - 1) / kTokens - (int64_t)r.blocks.size() + (cow ? 1 : 0);
  if (need > num_free_) return -3;
  *num_copies = 0;
  if (cow) {
    const int32_t old = r.blocks.back();
    const int32_t fresh = take_head();
    --blocks_[old].ref;
    r.blocks.back() = fresh;
    copy[0] = old;
    copy[1] = fresh;
    *num_copies = 1;
  }
  while ((int64_t)r.blocks.size() * kTokens < T + n) r.blocks.push_back(take_head());
  for (int32_t i = 0; i < n; ++i) {
    const int64_t t = T + i;
    slots[i] = (int64_t)r.blocks[t / kTokens] * kTokens + t % kTokens;
  }
  r.tokens.insert(r.tokens.end(), tokens, tokens + n);
  // index the blocks this call filled
  const int64_t total = (int64_t)r.tokens.size();
  for (int64_t j = T / kTokens; j < total / kTokens; ++j) {
    Block& k = blocks_[r.blocks[j]];
    if (k.keyed) continue;
    const uint64_t parent = j == 0 ? kRoot : blocks_[r.blocks[j - 1]].hash;
    const int32_t* toks = r.tokens.data() + j * kTokens;
    const uint64_t h = chain_hash(parent, toks);
    // the hash of an indexed block is always that of its content; a block
    // filled but not indexed (its content indexed elsewhere) still needs it
    // as the parent of the next block
    k.hash = h;
    k.parent_hash = parent;
    memcpy(k.tokens, toks, sizeof(k.tokens));
    if (index_.count(h)) continue;
    index_.emplace(h, r.blocks[j]);
    k.keyed = true;
  }
  return 0;
}

int BlockPool::fork(int64_t parent, int64_t child) {
  auto it = reqs_.find(parent);
  if (it == reqs_.end()) return -1;
  if (reqs_.count(child)) return -2;
  Request c = it->second;
  for (int32_t b : c.blocks) ++blocks_[b].ref;
  reqs_.emplace(child, std::move(c));
  return 0;
}

int BlockPool::free_request(int64_t req) {
  auto it = reqs_.find(req);
  if (it == reqs_.end()) return -1;
  const std::vector<int32_t>& bl = it->second.blocks;
  for (auto b = bl.rbegin(); b != bl.rend(); ++b)
    if (--blocks_[*b].ref == 0) queue_push_tail(*b);
  reqs_.erase(it);
  return 0;
}

const std::vector<int32_t>* BlockPool::table(int64_t req) const {
  auto it = reqs_.find(req);
  return it == reqs_.end() ? nullptr : &it->second.blocks;
}

int32_t BlockPool::num_tokens(int64_t req) const {
  auto it = reqs_.find(req);
  return it == reqs_.end() ? -1 : (int32_t)it->second.tokens.size();
}

}  // namespace pa
