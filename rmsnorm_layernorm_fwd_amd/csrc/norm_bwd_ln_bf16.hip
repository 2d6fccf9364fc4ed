// norm_bwd_ln_bf16.hip -- backward row kernels instantiated for one
// (type, operator, epilogue) combination; see norm_bwd.hpp and
// norm_bwd_long.hpp.
#include "norm_bwd.hpp"
#include "norm_bwd_long.hpp"

namespace nr {
NR_BWD_INSTANTIATE(bf16, true, kEpiNone)
NR_BWD_LONG_INSTANTIATE(bf16, true, kEpiNone)
}  // namespace nr
