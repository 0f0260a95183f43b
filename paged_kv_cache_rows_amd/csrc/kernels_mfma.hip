// MFMA part kernel for many query vectors per KV head (rows * group >= 16): not built yet.
#include "internal.h"

namespace kvp {

int mfma_chunk(int D) { return D == 512 ? 256 : 512; }
bool mfma_supported(int, int, int) { return false; }
int mfma_query_tiles(int, int, int) { return 1; }
hipError_t launch_part_mfma(int, int, const PartArgs &, int, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace kvp
