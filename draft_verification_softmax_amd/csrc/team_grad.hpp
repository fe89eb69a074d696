// team_grad.hpp -- gradient of the end-to-end TV objective in the drafter logits, computed by
// teams of workgroups (one team per row pair, as in the verification stream kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "team.hpp"

namespace sv {

struct GradArgs {
    void *grad;             // [rows][ld_g] gradient rows, dtype_g
    int64_t ld_g;
    const float *alpha;     // [I][D] overlaps of the same inputs
    const float *grad_loss; // device scalar, or null for 1
    float *scale;           // [rows] workspace: -grad_loss * w_{i,k} / (|I| D T)
    double inv_idt;         // 1 / (|I| D T)
};

// Weights kernel, team gradient kernel and fix-up kernel, in stream order.  a: as for the
// L_e2e forward (B = |I|, K = slots = trows = D); the epoch advances at the end.
hipError_t team_launch_grad(const TeamArgs &a, const GradArgs &g, int dtype_t, int dtype_d, int dtype_g,
                            hipStream_t s);

}  // namespace sv
