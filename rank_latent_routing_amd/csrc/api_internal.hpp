// Host-side helpers of the C ABI shared between its source files (not part
// of the public surface, include/flare.h).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/flare.h"

namespace flare {

// Every check flare_encode makes except those on its workspace: FLARE_OK, or
// the status flare_encode would return for these arguments.
flare_status encode_validate(const flare_tensor* Q, const flare_tensor* K, const flare_tensor* V,
                             const flare_tensor* Z, const float* lse, int B, int H, int M, int64_t N,
                             int D, float scale, unsigned flags);

// The largest token-split count, at most the planner's own choice, whose
// partial results fit in max_bytes of workspace; 0 if one split does not fit.
int encode_splits_within(int B, int H, int M, int64_t N, int D, int is_f32, size_t max_bytes);

// A validated encoder call with its split partials in ws, the splits capped at
// max_splits (0: the planner's choice, the size flare_encode_workspace_size
// reports).  The merge reads only what the split kernel writes in the same
// call, so ws needs no clearing.
flare_status encode_run(const flare_tensor* Q, const flare_tensor* K, const flare_tensor* V,
                        const flare_tensor* Z, float* lse, int B, int H, int M, int64_t N, int D,
                        float scale, unsigned flags, void* ws, int max_splits, void* stream);

}  // namespace flare
