// norm_bwd_gelu_f32.hip -- backward row kernels instantiated for one
// (type, operator, epilogue) combination; see norm_bwd.hpp.
#include "norm_bwd.hpp"

namespace nr {
NR_BWD_INSTANTIATE(float, true, kEpiGelu)
}  // namespace nr
