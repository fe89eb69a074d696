// team_sample.hpp -- draft tokens and their confidences from the drafter rows, computed by
// teams of workgroups (one team per drafter row) and, in the same launch, one finalize wave
// per row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "team.hpp"

namespace sv {

// a: B requests x K drafter rows (slots = K), draft / ld_d / c / seed / step set; tokens and
// conf are [B][K].  Greedy when a.c == 0.  The epoch advances at the end.
hipError_t team_launch_sample(const TeamArgs &a, int dtype_d, int32_t *tokens, float *conf, hipStream_t s);

}  // namespace sv
