// The merge kernel: the exact LSE merge of partial attention states (device
// code in merge_device.hpp) as its own launch. Each wave merges one unit (a
// run of consecutive output rows of one request), or each work-group one unit
// with many states. The kernel is a pure HBM stream: every state vector is
// read once, coalesced, and every output row written once.
#include "merge_device.hpp"

namespace skv {

// kMany: one work-group per unit, its four waves taking R-row steps in turn
// (finer pieces than a wave per unit, so the grid ends evenly); otherwise one
// wave per unit, row by row (units of a few rows: decode merges of many
// splits, where a work-group per unit would leave most waves idle).
template <int DV, bool kMany>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int unit = kMany ? blockIdx.x : blockIdx.x * 4 + wave;
  if (unit >= a.num_units) return;
  const DevUnit u = a.units[unit];
  const DevReq rq = a.reqs[u.b];
  const int S = rq.splits + a.n_ext;  // <= 64 + n_ext, at most 128 (host-checked)
  if (kMany) {
    if (S > kFew) {
      merge_rows_many<DV>(a, u, rq, S, lane, R * wave, 4 * R);
      return;
    }
    if (wave != 0) return;   // a few-state unit: one wave, as below
  }

  merge_rows_wave<DV>(a, u, rq, S, lane);
}

hipError_t launch_merge(const MergeLaunch& m) {
  if (m.num_units == 0) return hipSuccess;
  const MergeArgs a = merge_args(m);
  // the many-state shape needs units of at least R rows (each wave takes R)
  const bool many = m.max_states > kFew && m.run >= R;
  const dim3 grid(many ? m.num_units : (m.num_units + 3) / 4), block(256);
  switch (m.head_dim_v) {
    case 64:
      if (many) hipLaunchKernelGGL((merge_kernel<64, true>), grid, block, 0, m.stream, a);
      else hipLaunchKernelGGL((merge_kernel<64, false>), grid, block, 0, m.stream, a);
      break;
    case 128:
      if (many) hipLaunchKernelGGL((merge_kernel<128, true>), grid, block, 0, m.stream, a);
      else hipLaunchKernelGGL((merge_kernel<128, false>), grid, block, 0, m.stream, a);
      break;
    case 512:
      if (many) hipLaunchKernelGGL((merge_kernel<512, true>), grid, block, 0, m.stream, a);
      else hipLaunchKernelGGL((merge_kernel<512, false>), grid, block, 0, m.stream, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Before a fused launch: the merge's arguments into the block's header and
// every counter to zero, by a kernel (not a copy or a memset), so that the
// sequence can be captured in a HIP graph.
__global__ __launch_bounds__(256) void fused_setup_kernel(uint8_t* block, MergeArgs m, int n,
                                                         int num_tasks) {
  if (threadIdx.x == 0) *reinterpret_cast<MergeArgs*>(block) = m;
  int32_t* ctr = reinterpret_cast<int32_t*>(block + kFusedArgsBytes);
  for (int i = threadIdx.x; i < n; i += 256) ctr[i] = i == kFusedCounterLine ? num_tasks : 0;
}

hipError_t launch_fused_setup(uint8_t* block, const MergeLaunch& m, int batch, int num_tasks,
                              hipStream_t stream) {
  hipLaunchKernelGGL(fused_setup_kernel, dim3(1), dim3(256), 0, stream, block, merge_args(m),
                     (kFusedCounterHead + batch) * kFusedCounterLine, num_tasks);
  return hipGetLastError();
}

}  // namespace skv
