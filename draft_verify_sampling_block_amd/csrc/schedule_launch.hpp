// Launcher of the scheduler kernel (schedule.hip), shared by the three
// scheduler entry points of the C ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dspark {

// stop rules: Theta = tau * SPS rises; a fixed count K of candidates; a
// fixed survival threshold
constexpr int kSchedTheta = 0, kSchedCapacity = 1, kSchedThreshold = 2;

// mode kSchedTheta reads sps[0..sps_len); kSchedCapacity reads capacity[0]
// (device fp64) when the kernel runs; kSchedThreshold compares with
// `threshold`.  Unused pointers may be NULL.
// `traced` false keeps the launches out of the optional tracer (which
// creates events).
hipError_t launch_schedule(int R, int gamma, const float* conf, const double* sps, int sps_len,
                           int mode, double threshold, const double* capacity, int32_t* ell,
                           int32_t* order, double* stats, int32_t* status, void* ws,
                           hipStream_t stream, bool traced = true);

// The allocation-free entry point's scratch (the ranks): its size, and its
// device address on the current device (looked up once per device; NULL
// with *err set when the lookup fails).
size_t schedule_scratch_bytes();
int32_t* schedule_scratch(hipError_t* err);

}  // namespace dspark
