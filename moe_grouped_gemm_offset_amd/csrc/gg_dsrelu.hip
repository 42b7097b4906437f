// gg_dsrelu.hip -- launcher of the block-scaled dgrad + dsReLU kernels
// (gg_dsrelu.hpp): B's major selects the object whose kernels run.
#include "gg_dsrelu.hpp"

namespace gg {

// The kernels' dtype codes are the ABI's gg_dtype values.
static_assert(kBF16 == GG_BF16 && kF16 == GG_F16 && kF32 == GG_F32 && kF8 == GG_F8E4M3 &&
                  kF8E5M2 == GG_F8E5M2,
              "dtype codes");

hipError_t launch_dsrelu(const DsreluArgs& p, hipStream_t s, LaunchInfo* info) {
    using C = DsreluCfg;
    const int64_t tiles = ((p.m_rows + C::TM - 1) / C::TM) * ((p.N + C::TN - 1) / C::TN);
    if (tiles == 0)
        return hipSuccess;
    if (info) {
        snprintf(info->kernel, sizeof(info->kernel), "dsrelu_kernel<A/B %s, B %s-major, C %s, D %s>",
                 p.ab_e5m2 ? "e5m2" : "e4m3", p.b_kmajor ? "K" : "N", dtype_name(p.c_dtype),
                 dtype_name(p.d_dtype));
        info->tm = C::TM;
        info->tn = C::TN;
        info->waves = C::kWaves;
        info->grid = tiles;
    }
    return p.b_kmajor ? launch_dsrelu_bk<true>(p, s) : launch_dsrelu_bk<false>(p, s);
}

}  // namespace gg
