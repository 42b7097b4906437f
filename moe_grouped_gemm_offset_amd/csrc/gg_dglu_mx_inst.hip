// gg_dglu_mx_inst.hip -- the block-scaled dgrad + dGLU kernels of one
// activation (GG_ACT: 0 dSwiGLU, 1 dGeGLU, 2 dSiTU-GLU) and B major (GG_BK:
// 1 K-major, 0 N-major), both set by the build, one object per pair.
#include "gg_dglu_mx.hpp"

namespace gg {

template hipError_t launch_dglu_mx_act<GG_ACT, GG_BK != 0>(const DgluArgs&, hipStream_t);

}  // namespace gg
