// Tiled-CSL product kernels, N padded to 64.

#include "lscd_skinny.h"

namespace lscd {

hipError_t launch_kind_skinny64(int kind, int R, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    return launch_spmm_n<64>(kind, R, a, grid, st, occ);
}

}  // namespace lscd
