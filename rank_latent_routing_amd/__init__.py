"""MI355X-native FLARE / FLARE++ low-rank token mixer.

The compute lives in a gfx950 HIP library with a plain C ABI
(include/flare.h): split-token encode with an exact logsumexp merge, a
decode with a per-token softmax over the latents, FLARE++ query synthesis,
and bf16 matrix-core projections.  This package holds the ctypes binding
(argument marshalling only), the library's build script, the seeded input
generators and the algorithmic cost model used for roofline accounting.
"""
from .binding import (  # noqa: F401
    FLARE_ACCUMULATE_DK, FLARE_ACCUMULATE_DQ, FLARE_BF16, FLARE_F32, FLARE_FLAG_EXACT_SOFTMAX, FLARE_MIX_FUSED_WO,
    FLARE_SUM_DQ_OVER_BATCH,
    FlareError, describe, encode_workspace_size, flare_decode, flare_decode_backward, flare_encdec_backward,
    flare_encode,
    flare_encode_backward, flare_mix, flare_project, flare_route_queries, lib, mix_workspace_size,
    project_workspace_size, status_string, token_major, version)
