// Host-side pool state shared by the pool bookkeeping (pool.cpp, no HIP dependency) and
// the kernel launchers (which read the layout and the region table).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "kvattn.h"

struct kvattn_pool {
  kvattn_layout layout;
  int64_t block_bytes = 0;
  int32_t n_regions = 0;
  void* base[KVATTN_MAX_REGIONS] = {};
  int64_t first_id[KVATTN_MAX_REGIONS + 1] = {};  // first_id[n_regions] = total blocks
  int64_t total_blocks = 0;
  std::vector<int32_t> free_stack;  // next block handed out = back()
  std::vector<int32_t> refcount;
  int64_t shared_blocks = 0;        // blocks with refcount >= 2
  int32_t borrowers = 0;            // placement stores holding this pool
  bool free_requested = false;      // kvattn_pool_free called while borrowed
};

namespace kvattn {
// A placement store takes / gives back a pool; giving back the last borrow of a pool whose
// free was requested deletes it.
void pool_borrow(kvattn_pool* p);
void pool_unborrow(kvattn_pool* p);
// CPU tokens kvattn_share_admit would give, without admitting (-1 if already admitted).
int64_t share_admit_tokens(const kvattn_share_ctl* ctl, int64_t prefill_tokens,
                           int64_t block_tokens);
}  // namespace kvattn

namespace kvattn {

// Thread-local last-error message; set_error returns `code` for convenient returns.
kvattn_status set_error(kvattn_status code, const std::string& msg);
void clear_error();

// Layout checks shared by the pool and the launchers; returns an empty string when valid.
std::string layout_problem(const kvattn_layout& l);

inline int32_t elem_bytes(int32_t dtype) { return dtype == KVATTN_F32 ? 4 : 2; }

}  // namespace kvattn
