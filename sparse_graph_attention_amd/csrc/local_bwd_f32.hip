// fp32 instantiations of the local attention backward kernels.
#define GGA_BWD_IMPL
#include "local_bwd_impl.hpp"

namespace gga {
bool launch_bwd_f32(const BwdParams& p, int epl, int hdp, int ns, int mode, unsigned grid_a, unsigned grid_b,
                    int64_t max_heavy, hipStream_t s) {
    return launch_bwd_dtype<float, 4>(p, epl, hdp, ns, mode, grid_a, grid_b, max_heavy, s);
}
}  // namespace gga
