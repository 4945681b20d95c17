// Status codes and version string of the C ABI.
#include <stdio.h>

#include "common.h"

namespace quads {
namespace {
thread_local char g_last_hip[256];
}

int set_hip_error(hipError_t e) {
    snprintf(g_last_hip, sizeof g_last_hip, "HIP error %d: %s", (int)e, hipGetErrorString(e));
    return QUADS_EHIP;
}
}  // namespace quads

extern "C" const char* quads_status_string(int status) {
    switch (status) {
        case QUADS_OK: return "ok";
        case QUADS_EINVAL: return "invalid argument (null or misaligned pointer, or bad enum)";
        case QUADS_ESHAPE: return "invalid shape (see the size rules in quads.h)";
        case QUADS_EWORKSPACE: return "workspace too small (query the matching *_ws function)";
        case QUADS_EHIP: return quads::g_last_hip[0] ? quads::g_last_hip : "HIP error";
        case QUADS_ESCRATCH:
            return "input too large for the static scratch of a no-allocation call "
                   "(quads_rac_quantize_ws exceeds QUADS_RAC_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

extern "C" const char* quads_version(void) { return "quads-mi355x 0.1 gfx950"; }
