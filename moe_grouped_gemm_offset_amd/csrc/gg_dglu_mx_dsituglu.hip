// gg_dglu_mx_dsituglu.hip -- the block-scaled dgrad + dSiTU-GLU kernels (gg_dglu_mx.hpp),
// in a translation unit of their own.
#include "gg_dglu_mx.hpp"

namespace gg {

template hipError_t launch_dglu_mx_act<2>(const DgluArgs&, hipStream_t);

}  // namespace gg
