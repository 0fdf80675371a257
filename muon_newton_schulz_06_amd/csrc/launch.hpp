// Launch wrappers implemented in the .hip translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <string>

#include "common.hpp"

namespace muon {

// GEMM-shaped products; `tile` is the square workgroup tile (128 or 256).
hipError_t launch_gemm(int op, int tile, const GemmLaunch& L, int blocks, hipStream_t st);
// Momentum + partial sums of squares, or partial sums of squares alone.
hipError_t launch_ew(const EwLaunch& L, int64_t blocks, hipStream_t st);
// alpha[i] = 1 / (sqrt(sum of partials) + eps), one workgroup per matrix.
hipError_t launch_norm(const NormLaunch& L, hipStream_t st);
// Scaled cast into the two operand layouts (and zero padding).
hipError_t launch_cast(const CastLaunch& L, int64_t blocks, hipStream_t st);

// Momentum fused with the operand cast (elementwise.hip).
hipError_t launch_momcast(const MomCastLaunch& L, int64_t blocks, hipStream_t st);

// Selected-row step: B = M + g with row scores; top-k per matrix; gather of
// the selected block; scatter of the update and the buffer decay.
hipError_t launch_sel_accum(const SelLaunch& L, int64_t blocks, hipStream_t st);
hipError_t launch_sel_topk(const SelLaunch& L, hipStream_t st);
hipError_t launch_sel_gather(const SelLaunch& L, int64_t blocks, hipStream_t st);
hipError_t launch_sel_gather_cast(const SelCastLaunch& L, int64_t blocks, hipStream_t st);
hipError_t launch_sel_scatter(const SelLaunch& L, int64_t blocks, hipStream_t st);

// Library state shared across translation units (implemented in api.cpp):
// the calling thread's last-error message, and whether calls made by this
// thread may use events and streams the library creates (profiling events,
// concurrent lanes); off for the entry point that allocates nothing.
void set_last_error(const std::string& msg);
void set_no_events(bool on);

}  // namespace muon
