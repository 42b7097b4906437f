// gg_dsrelu_inst.hip -- the block-scaled dgrad + dsReLU kernels of one B
// major (GG_BK: 1 K-major, 0 N-major; set by the build, one object each).
#include "gg_dsrelu.hpp"

namespace gg {

template hipError_t launch_dsrelu_bk<GG_BK != 0>(const DsreluArgs&, hipStream_t);

}  // namespace gg
