// Version and status strings of the C ABI.
#include "common.hpp"

extern "C" int gga_abi_version(void) { return GGA_ABI_VERSION; }

extern "C" const char* gga_status_string(int status) {
    switch (status) {
        case GGA_OK: return "ok";
        case GGA_EINVAL: return "invalid argument";
        case GGA_ERANGE: return "size out of range";
        case GGA_EUNSUPPORTED: return "unsupported dtype, mode or shape";
        case GGA_EWORKSPACE: return "workspace or plan buffer too small";
        case GGA_EHIP: return "HIP runtime error";
        case GGA_ESCRATCH: return "input needs more scratch than the allocation-free entry point's fixed array";
        default: return "unknown status";
    }
}
