// Tiled-CSL product kernels, N padded to 16.

#include "lscd_skinny.h"

namespace lscd {

hipError_t launch_kind_skinny16(int kind, int R, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    return launch_spmm_n<16>(kind, R, a, grid, st, occ);
}

}  // namespace lscd
