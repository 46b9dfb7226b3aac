// Dynamic request batcher: forms jagged batches of up to max_batch requests
// from a stream of arrivals ("NVIDIA Dynamo-Triton Gets End-to-End HSTU
// Generative Recommender Workflow", section Five stages and the benchmark:
// the server runs at dynamic batch size 8; "HSTU生成式推荐系统部署实战：NVIDIA
// Dynamo-Triton详解", Triton section: dynamic batching of variable-length
// sequences).  The pages give no policy; the one here is the usual
// size-or-delay rule, plus the constraint the KV cache imposes (one request
// per user in a batch), stated in hstu.h.
#include <algorithm>
#include <deque>
#include <unordered_set>

#include "internal.h"

using hstu::fail;
using hstu::ok;

struct hstu_batcher {
  struct Req {
    int64_t id, user;
    int32_t n_new;
    int64_t arrival_us;
  };
  int32_t max_batch = 8;
  int64_t max_delay_us = 0;
  int64_t max_tokens = 0;
  std::deque<Req> queue;
};

namespace {
// The batch the queue would give now: queue positions, FIFO, skipping
// requests of a user already taken; `full` when no further request can join.
std::vector<size_t> candidate(const hstu_batcher* b, bool* full) {
  std::vector<size_t> pick;
  std::unordered_set<int64_t> users;
  int64_t tokens = 0;
  *full = false;
  for (size_t i = 0; i < b->queue.size(); ++i) {
    const auto& r = b->queue[i];
    if (users.count(r.user)) continue;
    if (b->max_tokens > 0 && !pick.empty() && tokens + r.n_new > b->max_tokens) {
      *full = true;
      break;
    }
    pick.push_back(i);
    users.insert(r.user);
    tokens += r.n_new;
    if (static_cast<int32_t>(pick.size()) == b->max_batch) {
      *full = true;
      break;
    }
  }
  return pick;
}
}  // namespace

extern "C" {

hstu_status hstu_batcher_create(const hstu_batcher_desc* d, hstu_batcher** out) {
  if (!d || !out) return fail(HSTU_ERR_INVALID, "hstu_batcher_create: null argument");
  *out = nullptr;
  if (d->max_batch < 1 || d->max_delay_us < 0 || d->max_tokens < 0)
    return fail(HSTU_ERR_INVALID, "hstu_batcher_create: max_batch >= 1, max_delay_us >= 0, max_tokens >= 0");
  auto* b = new hstu_batcher();
  b->max_batch = d->max_batch;
  b->max_delay_us = d->max_delay_us;
  b->max_tokens = d->max_tokens;
  *out = b;
  return ok();
}

hstu_status hstu_batcher_destroy(hstu_batcher* b) {
  delete b;
  return ok();
}

hstu_status hstu_batcher_submit(hstu_batcher* b, int64_t request_id, int64_t user, int32_t n_new,
                                int64_t arrival_us) {
  if (!b || n_new < 0) return fail(HSTU_ERR_INVALID, "hstu_batcher_submit: bad arguments");
  b->queue.push_back(hstu_batcher::Req{request_id, user, n_new, arrival_us});
  return ok();
}

hstu_status hstu_batcher_next(hstu_batcher* b, int64_t now_us, int64_t* request_ids, int32_t cap, int32_t* n,
                              int64_t* wait_us) {
  if (!b || !n || !wait_us || cap < 0 || (cap > 0 && !request_ids))
    return fail(HSTU_ERR_INVALID, "hstu_batcher_next: bad arguments");
  *n = 0;
  if (b->queue.empty()) {
    *wait_us = -1;
    return ok();
  }
  bool full = false;
  std::vector<size_t> pick = candidate(b, &full);
  const int64_t waited = now_us - b->queue.front().arrival_us;
  if (!full && waited < b->max_delay_us) {
    *wait_us = b->max_delay_us - waited;
    return ok();
  }
  if (static_cast<int64_t>(pick.size()) > cap) return fail(HSTU_ERR_INVALID, "hstu_batcher_next: cap too small");
  for (size_t k = 0; k < pick.size(); ++k) request_ids[k] = b->queue[pick[k]].id;
  std::deque<hstu_batcher::Req> rest;
  size_t k = 0;
  for (size_t i = 0; i < b->queue.size(); ++i) {
    if (k < pick.size() && pick[k] == i) {
      ++k;
      continue;
    }
    rest.push_back(b->queue[i]);
  }
  b->queue.swap(rest);
  *n = static_cast<int32_t>(pick.size());
  *wait_us = 0;
  return ok();
}

hstu_status hstu_batcher_pending(const hstu_batcher* b, int32_t* n) {
  if (!b || !n) return fail(HSTU_ERR_INVALID, "hstu_batcher_pending: bad arguments");
  *n = static_cast<int32_t>(b->queue.size());
  return ok();
}

}  // extern "C"
