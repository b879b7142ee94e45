// Work-list planning for paged decode attention: one work-group of 1024
// threads runs the plan body (plan_body.h), which documents the work lists.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"
#include "plan_body.h"

namespace pkv {

namespace {

__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(PlanArgs a) {
  plan_body<kPlanThreads, kPlanMaxSeqs, kPlanMaxTasks, kMaxPartitions>(a);
}

}  // namespace

hipError_t launch_decode_plan(const PlanArgs& a, hipStream_t stream) {
  decode_plan_kernel<<<dim3(1), dim3(kPlanThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace pkv
