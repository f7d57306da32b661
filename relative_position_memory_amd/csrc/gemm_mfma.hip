#include "gemm_common.h"
namespace txl {
bool gemm_mfma_supported(const GemmArgs&) { return false; }
hipError_t launch_gemm_mfma(const GemmArgs&, hipStream_t) { return hipErrorInvalidValue; }
}
