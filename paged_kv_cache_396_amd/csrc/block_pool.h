// Host-side KV block pool: which physical blocks hold which request's tokens.
//
// The policy (pages cited by title and section):
//  * blocks are shared between requests through reference counts; a request
//    that must write into a partly filled block someone else still holds
//    gets a copy of it first (zihan-zhang.net vLLM study, 3.2.2: sharing and
//    copy-on-write; plumephp.com vLLM deep dive, 4.2);
//  * every full block is indexed by a prefix-cumulative hash: its parent's
//    hash combined with its own 16 tokens, so a match means the whole prefix
//    matches (same page, 3.6.1).  A hash hit is confirmed by comparing the
//    stored parent hash and tokens;
//  * freed blocks keep their hash and join the tail of a doubly linked free
//    queue; allocation takes the head (least recently used) and only then
//    drops the block's old hash from the index (same page, 3.6.2 and 5.5);
//  * a new request first collects its prompt's cached blocks up to the first
//    miss; allocation that cannot be served changes nothing (same page, 5.5);
//  * block 0 is a placeholder that is never handed out (same page, 5.5).
// Where the pages are silent: the first free queue holds blocks 1 .. N-1 in
// ascending order; the prompt lookup stops before the block holding the
// prompt's last token; a request's blocks are released last block first;
// a newly filled block whose content is already indexed is not indexed
// again.
//
// Not thread-safe: one caller at a time per pool.
#pragma once

#include <stdint.h>

#include <unordered_map>
#include <vector>

namespace pa {

class BlockPool {
 public:
  static constexpr int kTokens = 16;  // tokens per block

  explicit BlockPool(int32_t num_blocks);

  int32_t num_blocks() const { return (int32_t)blocks_.size(); }
  int32_t num_free() const { return num_free_; }

  // Status values: 0 ok, -1 unknown request, -2 request exists, -3 no free
  // blocks (nothing changed).
  int add_request(int64_t req, const int32_t* prompt, int32_t n, int32_t* num_cached);
  // Slots for the request's next n tokens (ids `tokens`); at most one
  // (src, dst) copy-on-write pair is returned through copy[0..1].
  int allocate_slots(int64_t req, const int32_t* tokens, int32_t n, int64_t* slots,
                     int32_t* copy, int32_t* num_copies);
  int fork(int64_t parent, int64_t child);
  int free_request(int64_t req);
  const std::vector<int32_t>* table(int64_t req) const;
  int32_t num_tokens(int64_t req) const;

 private:
  struct Block {
    int32_t ref = 0;
    int32_t prev = -1, next = -1;  // free-queue links
    bool in_free = false;
    bool keyed = false;            // full and present in the index
    uint64_t hash = 0, parent_hash = 0;
    int32_t tokens[kTokens];
  };
  struct Request {
    std::vector<int32_t> blocks;
    std::vector<int32_t> tokens;  // ids of the tokens that have slots
  };

  static uint64_t chain_hash(uint64_t parent, const int32_t* tokens);
  int32_t lookup(uint64_t parent, const int32_t* tokens) const;
  void queue_remove(int32_t b);
  void queue_push_tail(int32_t b);
  int32_t take_head();

  std::vector<Block> blocks_;
  int32_t head_ = -1, tail_ = -1, num_free_ = 0;
  std::unordered_map<uint64_t, int32_t> index_;
  std::unordered_map<int64_t, Request> reqs_;
};

}  // namespace pa
