// Tiled-CSL product kernels, N padded to 32.

#include "lscd_skinny.h"

namespace lscd {

hipError_t launch_kind_skinny32(int kind, int R, const SpmmArgs& a, int grid, hipStream_t st, int* occ) {
    return launch_spmm_n<32>(kind, R, a, grid, st, occ);
}

}  // namespace lscd
