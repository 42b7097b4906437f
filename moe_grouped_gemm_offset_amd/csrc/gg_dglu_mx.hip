// gg_dglu_mx.hip -- launcher of the block-scaled dgrad + dGLU kernels: the
// activation and B's major select the object (gg_dglu_mx_inst.hip, built
// once per pair) whose kernels run.
#include "gg_dglu_mx.hpp"

namespace gg {

hipError_t launch_dglu_mx(const DgluArgs& p, hipStream_t s, LaunchInfo* info) {
    using C = DgluMxCfg;
    const int64_t tiles = ((p.m_rows + C::TM - 1) / C::TM) * ((p.N + C::TN - 1) / C::TN);
    if (tiles == 0)
        return hipSuccess;
    if (info) {
        static const char* const kAct[] = {"dSwiGLU", "dGeGLU", "dSiTU-GLU"};
        snprintf(info->kernel, sizeof(info->kernel),
                 "dglu_mx_kernel<%s, A/B %s, B %s-major, C %s, D %s%s>", kAct[p.act],
                 p.ab_e5m2 ? "e5m2" : "e4m3", p.b_kmajor ? "K" : "N", dtype_name(p.c_dtype),
                 dtype_name(p.d_dtype), p.dbias ? ", dbias" : "");
        info->tm = C::TM;
        info->tn = C::TN;
        info->waves = C::kWaves;
        info->grid = tiles;
    }
    if (p.b_kmajor) {
        if (p.act == 0)
            return launch_dglu_mx_act<0, true>(p, s);
        if (p.act == 1)
            return launch_dglu_mx_act<1, true>(p, s);
        return launch_dglu_mx_act<2, true>(p, s);
    }
    if (p.act == 0)
        return launch_dglu_mx_act<0, false>(p, s);
    if (p.act == 1)
        return launch_dglu_mx_act<1, false>(p, s);
    return launch_dglu_mx_act<2, false>(p, s);
}

}  // namespace gg
