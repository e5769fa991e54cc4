// resident.hpp -- the split form of the resident-state substep: the grid
// update of the node tiles a deposit flagged, and the grid-to-particle
// gather over the binned records in place (grid.hip); the deposit is the
// fused kernel's deposit-only launch (fused.hip).
#pragma once
#include "common.hpp"

namespace mpmk {

hipError_t launch_grid_update_tiles(int dim, int n, int64_t *grid, uint8_t *tiles, float *vg, float dt,
                                    const float *gravity, int sticky, hipStream_t s);
hipError_t launch_g2p_records(int dim, int n, const BinView &b, const float *vg, float dt, uint32_t *status,
                              hipStream_t s);

}  // namespace mpmk
