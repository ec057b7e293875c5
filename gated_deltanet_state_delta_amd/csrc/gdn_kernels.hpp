// gdn_kernels.hpp -- internal launch entry points behind the C ABI.
//
// The C ABI (gdn_api.cpp) validates arguments and then calls these; each
// returns the hipError_t of its launch.  Arguments are already checked.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/libgdn.h"

namespace gdn {

hipError_t launch_gate(const float* A_log, const float* dt_bias, const void* a, const void* b,
                       int ab_dtype, int64_t n_tokens, int hv, float* log_decay, float* gamma,
                       float* beta, hipStream_t stream);

hipError_t launch_decode(const gdn_decode_args& args, hipStream_t stream);

// pool_flags (internal): the decode's rules when a multi-token decode runs as
// a pooled prefill -- kPoolSkipUnread: a request whose read slot is outside
// the pool is skipped entirely (no output, no state); kPoolNoWrite: no state
// is stored.
constexpr int kPoolSkipUnread = 1, kPoolNoWrite = 2;
hipError_t launch_prefill(const gdn_prefill_args& args, hipStream_t stream, int pool_flags = 0);

// Scratch bytes launch_prefill uses for these arguments when the workspace
// holds at least that many (the scan over segment maps); 0 when it needs none.
size_t prefill_workspace_bytes(const gdn_prefill_args& args);
// Reads (and optionally clears) the current device's count of expired
// in-kernel waits; synchronous.
hipError_t wait_timeouts(uint32_t* count, bool clear);

hipError_t launch_conv1d(const gdn_conv1d_args& args, hipStream_t stream);

}  // namespace gdn
