// Launches of the Gram-space A² products (kernel templates in gemm.hpp).
#include "gemm.hpp"

namespace muon {
template hipError_t launch_epi<EPI_SQ>(int, int, const GemmLaunch&, int, hipStream_t);
}  // namespace muon
