// Status strings of the C ABI.
#include "../../include/specv.h"

extern "C" const char* specv_status_string(int status) {
    switch (status) {
        case SPECV_OK: return "ok";
        case SPECV_E_INVAL: return "invalid argument";
        case SPECV_E_SHAPE: return "size outside the supported range";
        case SPECV_E_ALIGN: return "misaligned pointer";
        case SPECV_E_HIP: return "HIP launch failed";
        case SPECV_E_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}
