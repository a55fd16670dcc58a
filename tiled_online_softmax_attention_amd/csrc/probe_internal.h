// probe_internal.h -- launcher of the matrix-core rate probe, shared between
// the C-ABI host code (attn_api.hip) and probe_gfx950.hip.  Not installed;
// the public interface is include/attn.h.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

// Placements of the probe loop in instruction memory (see probe_gfx950.hip).
constexpr int kProbePlacements = 16;

// 0 on success, -1 launch failure.  Arguments are validated by the caller
// (placement in [0, kProbePlacements)).
int launch_mfma_probe(const void* fragments, int n_fragments, float* out, int blocks, int iters, int placement,
                      hipStream_t stream);

}  // namespace attn
