// Launches of the Gram-space a·Y + B·Y products (kernel templates in gemm.hpp).
#include "gemm.hpp"

namespace muon {
template hipError_t launch_epi<EPI_AXPY>(int, int, const GemmLaunch&, int, hipStream_t);
}  // namespace muon
