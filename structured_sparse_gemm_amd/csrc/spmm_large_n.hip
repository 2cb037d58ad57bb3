#include "ssg_kernels.hpp"
namespace ssg {
bool supported_large_n(const SpmmArgs&) { return false; }
hipError_t launch_spmm_large_n(const SpmmArgs&, hipStream_t) { return hipErrorInvalidValue; }
}
