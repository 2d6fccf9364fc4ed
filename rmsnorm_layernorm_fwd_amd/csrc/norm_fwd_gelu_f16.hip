// norm_fwd_gelu_f16.hip -- forward row kernels instantiated for one
// (type, operator, epilogue) combination; see norm_fwd.hpp.
#include "norm_fwd.hpp"

namespace nr {
NR_FWD_INSTANTIATE(f16, true, kEpiGelu)
}  // namespace nr
