// stress.hpp -- the elastic substep's F update and the next substep's
// stressed affine matrix in one pass over the particles (stress.hip).
#pragma once
#include "common.hpp"

namespace mpmk {

hipError_t launch_update_F_stress(int dim, int n, int64_t np, const float *C, float *F, const float *m,
                                  const float *vol0, float dt, float mu, float lambda, float *Cout, uint32_t *status,
                                  hipStream_t s);

}  // namespace mpmk
