// Fused attention-and-merge launch (LiquidCP section 6.2 and appendix A.3:
// CTAs switch from attention to reduction work after their last attention
// task; per-destination counters tell a reduction when its inputs are
// complete).
//
// The grid is the attention kernel's own: one work-group per task in the
// plan's queue order, each counting itself as started when it begins. After
// its task's partial state is stored, the work-group publishes it: every wave
// waits for its stores, the work-group meets at a barrier, and one thread adds
// 1 to the request's counter with an agent-scope release (on gfx950 a
// write-back of the XCD's L2 precedes the atomic, so the state has reached the
// coherence point). Then, if every task of the launch has started, the
// work-group turns to reduction: each wave claims merge units in queue order,
// polls the unit's request counter (relaxed coherent loads) until all its
// tasks have published, and merges the unit reading the partial states with
// coherent loads as well. Within a launch each partial state is written once
// and read only by its merge, so no reader holds a stale copy to invalidate.
// A work-group that finishes while some task has not started leaves instead,
// so a waiting wave never holds a slot that an unstarted task needs: every
// task a merge waits for is resident or done, and every wait ends. At least
// the last task to start takes the reduction role, so every unit is merged.
// Each wait is still bounded and reports through the error flag.
//
// The block (the scratch's counters block, written by fused_setup before
// every launch): the merge's arguments (MergeArgs, read only after the task,
// so that they occupy no registers while it runs), then int32 counters, each
// in a 256-byte line of its own (waves polling one line while others update
// a neighbour on it slowed the launch by a third when they shared lines):
// next merge unit, the number of attention tasks, tasks started, then per
// request b the attention tasks that have published.
#pragma once

#include "merge_device.hpp"

namespace skv {

struct FusedArgs {
  uint8_t* block;
};

static_assert(sizeof(MergeArgs) <= kFusedArgsBytes, "merge arguments fit the block's header");
__device__ __forceinline__ int32_t* fused_counters(const FusedArgs& f) {
  return reinterpret_cast<int32_t*>(f.block + kFusedArgsBytes);
}
constexpr int kCtrLine = kFusedCounterLine;   // int32 per counter line
constexpr int kCtrUnit = 0, kCtrTasks = kCtrLine, kCtrStarted = 2 * kCtrLine;
__device__ __forceinline__ int32_t* request_counter(int32_t* ctr, int b) {
  return ctr + (kFusedCounterHead + b) * kCtrLine;
}
constexpr uint32_t kSpinLimit = 1u << 20;   // polls of ~2000 cycles (after 16 short ones): ~1 s

// Count this work-group's task as started (first thing in the kernel).
__device__ __forceinline__ void count_started(const FusedArgs& f) {
  if (threadIdx.x == 0) atomicAdd(&fused_counters(f)[kCtrStarted], 1);
}

// Whether every task of the launch has started (the same answer for every
// thread; slot: one int of LDS).
__device__ __forceinline__ bool all_started(const FusedArgs& f, int* slot) {
  if (threadIdx.x == 0) {
    int32_t* ctr = fused_counters(f);
    *slot = __hip_atomic_load(&ctr[kCtrStarted], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= ctr[kCtrTasks];
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*slot) != 0;
}

// Make the task's stored state visible to every XCD, then count the task.
__device__ __forceinline__ void publish_task(const FusedArgs& f, int b) {
  __builtin_amdgcn_s_waitcnt(0);   // this wave's stores have reached the L2
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(request_counter(fused_counters(f), b), 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// The reduction role of one wave: merge units in queue order until none is
// left, each after its request's attention tasks have all published.
template <int DV>
__device__ __forceinline__ void reduce_phase(const FusedArgs& f, int32_t* err_flag) {
  const int lane = threadIdx.x & 63;
  int32_t* ctr = fused_counters(f);
  const MergeArgs m = *reinterpret_cast<const MergeArgs*>(f.block);
  for (;;) {
    int u = 0;
    if (lane == 0) u = atomicAdd(&ctr[kCtrUnit], 1);
    u = __builtin_amdgcn_readfirstlane(u);
    if (u >= m.num_units) return;
    const DevUnit du = m.units[u];
    const DevReq rq = m.reqs[du.b];
    // poll with relaxed loads (coherent reads that leave the caches alone)
    bool ready = true;
    for (uint32_t spins = 0;; ++spins) {
      const int done = __hip_atomic_load(request_counter(ctr, du.b), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (done >= rq.tasks) break;
      if (spins >= kSpinLimit) {
        ready = false;
        break;
      }
      if (spins < 16) __builtin_amdgcn_s_sleep(2);
      else __builtin_amdgcn_s_sleep(31);
    }
    if (!ready) {
      if (lane == 0) raise_error(err_flag, kErrWait);
      merge_rows_nan<DV>(m, du, rq, lane);
      continue;
    }
    // the states are read with coherent loads (see StateIO): no acquire, whose
    // cache invalidation per unit would slow every wave of this XCD
    merge_rows_wave<DV, true>(m, du, rq, rq.splits + m.n_ext, lane);
  }
}

// Host side: kernel arguments of a fused launch.
inline FusedArgs fused_args(const FusedLaunch& F) {
  FusedArgs f;
  f.block = F.block;
  return f;
}

}  // namespace skv
