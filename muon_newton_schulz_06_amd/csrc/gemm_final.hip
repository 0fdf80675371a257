// Launches of the final products (weight update, plain output) and the
// dispatcher over every epilogue (kernel templates in gemm.hpp).
#include "gemm.hpp"

namespace muon {

template hipError_t launch_epi<EPI_UPDATE>(int, int, const GemmLaunch&, int, hipStream_t);
template hipError_t launch_epi<EPI_OUT>(int, int, const GemmLaunch&, int, hipStream_t);

hipError_t launch_gemm(int op, int tile, const GemmLaunch& L, int blocks, hipStream_t st) {
  if (blocks <= 0) return hipSuccess;
  const int epi = L.seg[0].epi;
  for (int k = 1; k < L.nseg; ++k)
    if (L.seg[k].epi != epi) return hipErrorInvalidValue;  // one epilogue per launch
  switch (epi) {
    case EPI_SYRK: return launch_epi<EPI_SYRK>(op, tile, L, blocks, st);
    case EPI_SQ: return launch_epi<EPI_SQ>(op, tile, L, blocks, st);
    case EPI_AXPY: return launch_epi<EPI_AXPY>(op, tile, L, blocks, st);
    case EPI_UPDATE: return launch_epi<EPI_UPDATE>(op, tile, L, blocks, st);
    case EPI_OUT: return launch_epi<EPI_OUT>(op, tile, L, blocks, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace muon
