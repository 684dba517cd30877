// Shared between the host update (zero_host_adam.cpp) and the offloaded step (zero_offload.cpp).
#pragma once

#include <condition_variable>
#include <mutex>
#include <thread>
#include <vector>

#include "zero_internal.h"

namespace zero {

struct HostStep;
typedef void (*HostRangeFn)(const HostStep&, uint64_t, uint64_t);

// A team of host threads that one call keeps for all of its updates (the offloaded step updates
// its shard chunk by chunk), so threads are started once per call, not once per chunk. The caller
// is the team's first member. Threads that cannot be started are simply left out; a team of one
// runs everything on the caller. No exception leaves the constructor or run().
class HostTeam {
 public:
  explicit HostTeam(uint32_t threads);
  ~HostTeam();
  HostTeam(const HostTeam&) = delete;
  HostTeam& operator=(const HostTeam&) = delete;
  uint32_t size() const { return (uint32_t)workers_.size() + 1; }
  // fn over [0, n), split as the per-call path splits it over size() threads
  void run(HostRangeFn fn, const HostStep& s, uint64_t n);

 private:
  void work(uint32_t member);
  std::mutex mu_;
  std::condition_variable go_, done_;
  std::vector<std::thread> workers_;
  uint64_t generation_ = 0;
  uint32_t pending_ = 0;
  bool stop_ = false;
  HostRangeFn fn_ = nullptr;
  const HostStep* step_ = nullptr;
  uint64_t n_ = 0, per_ = 0;
  uint32_t used_ = 1;   // members with a range in the current job
};

// Argument checks of the host update; need_grad: grad must be non-NULL when n > 0.
zero_status check_host_args(const char* fn, bool need_grad, const float* grad, uint64_t n,
                            float* master, float* m, float* v, const zero_adam_hparams* hp,
                            void* out, int32_t out_dtype, zero_adam_scalars* k);

// The update of [0, n) on host arrays with the given constants, split over `threads` threads
// started for this call, or over `team` when one is given.
zero_status host_step(const float* grad, uint64_t n, float grad_scale, float* master, float* m,
                      float* v, const zero_adam_scalars& k, bool l2, void* out, int out_dtype,
                      uint32_t threads, HostTeam* team = nullptr);

}  // namespace zero
