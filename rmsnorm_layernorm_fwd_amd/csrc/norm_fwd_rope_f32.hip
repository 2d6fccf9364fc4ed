// norm_fwd_rope_f32.hip -- forward row kernels instantiated for one
// (type, operator, epilogue) combination; see norm_fwd.hpp.
#include "norm_fwd.hpp"

namespace nr {
NR_FWD_INSTANTIATE(float, false, kEpiRope)
}  // namespace nr
