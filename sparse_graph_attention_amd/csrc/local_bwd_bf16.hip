// bf16 instantiations of the local attention backward kernels.
#define GGA_BWD_IMPL
#include "local_bwd_impl.hpp"

namespace gga {
bool launch_bwd_bf16(const BwdParams& p, int epl, int hdp, int ns, int mode, unsigned grid_a, unsigned grid_b,
                     int64_t max_heavy, hipStream_t s) {
    return launch_bwd_dtype<uint16_t, 8>(p, epl, hdp, ns, mode, grid_a, grid_b, max_heavy, s);
}
}  // namespace gga
