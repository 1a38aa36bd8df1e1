// prefill_wide.hip -- the tile kernel with two 32-row column blocks per wave
// (64 query rows): every K fragment feeds two S^T MFMAs and every V^T
// fragment two O^T MFMAs, so LDS fragment reads and the L2 -> LDS tile
// traffic per flop are half those of one block per wave.  One wave per SIMD
// (4 waves, 256 rows per workgroup, one workgroup per CU); the O^T
// accumulators need more than the 256 VGPRs a lane has, so this file is
// compiled without the VGPR-only MFMA form and the compiler places them in
// AGPRs.
#include "prefill_tile.h"

namespace pa {

hipError_t launch_prefill_wide(const AttnParams &p, hipStream_t stream, LaunchInfo *li) {
    switch (p.head_dim) {
        case 128: return launch_tiles<128, 64, 3, false, 4, 2>(p, stream, li);
        case 256: return launch_tiles<256, 32, 3, false, 4, 2>(p, stream, li);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
