// Entry points whose kernels are not written yet: they report GGA_EUNSUPPORTED.
#include "common.hpp"

extern "C" int gga_edge_values(int32_t, int32_t, int32_t, const void*, int64_t, const int32_t*, void*, void*) {
    return GGA_EUNSUPPORTED;
}
extern "C" int gga_edge_values_bwd(int32_t, int32_t, int64_t, const int32_t*, const int32_t*, const float*, float*,
                                   void*) { return GGA_EUNSUPPORTED; }
extern "C" int gga_gat_coef_fwd(int32_t, int32_t, int32_t, const float*, const float*, const float*, float*, float*,
                                void*) { return GGA_EUNSUPPORTED; }
extern "C" size_t gga_gat_coef_bwd_workspace(int32_t, int32_t, int32_t) { return 0; }
extern "C" int gga_gat_coef_bwd(int32_t, int32_t, int32_t, const float*, const float*, const float*, const float*,
                                const float*, const float*, float*, float*, float*, void*, size_t, void*) {
    return GGA_EUNSUPPORTED;
}
extern "C" int gga_linear(int32_t, int32_t, int32_t, int32_t, int32_t, const float*, const float*, const float*,
                          float*, void*) { return GGA_EUNSUPPORTED; }
extern "C" size_t gga_global_linear_workspace(int32_t, int32_t, int32_t) { return 0; }
extern "C" int gga_global_linear_fwd(int32_t, int32_t, int32_t, const float*, const float*, const float*, float,
                                     float*, float*, float*, void*, size_t, void*) { return GGA_EUNSUPPORTED; }
extern "C" int gga_gated_combine(int32_t, int32_t, const float*, const float*, float, int32_t, const float*,
                                 const float*, float*, float*, void*) { return GGA_EUNSUPPORTED; }
extern "C" int gga_add_layernorm(int32_t, int32_t, const float*, const float*, const float*, const float*, float,
                                 float*, void*) { return GGA_EUNSUPPORTED; }
