// Launches of the SYRK products (kernel templates in gemm.hpp).
#include "gemm.hpp"

namespace muon {
template hipError_t launch_epi<EPI_SYRK>(int, int, const GemmLaunch&, int, hipStream_t);
}  // namespace muon
