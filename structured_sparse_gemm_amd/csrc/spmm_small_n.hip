#include "ssg_kernels.hpp"
namespace ssg {
bool supported_small_n(const SpmmArgs&) { return false; }
hipError_t launch_spmm_small_n(const SpmmArgs&, hipStream_t) { return hipErrorInvalidValue; }
}
