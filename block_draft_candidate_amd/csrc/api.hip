// Status strings and version of libdflash.
#include "common.h"

extern "C" const char* dflash_status_string(int status) {
    switch (status) {
        case DFLASH_OK: return "ok";
        case DFLASH_ERR_INVALID_ARG: return "invalid argument (null/misaligned pointer or size out of range)";
        case DFLASH_ERR_UNSUPPORTED: return "unsupported size (see the call's requirements)";
        case DFLASH_ERR_WORKSPACE: return "workspace smaller than the size query returned";
        case DFLASH_ERR_HIP: return "HIP launch failure";
        case DFLASH_ERR_SCRATCH: return "problem needs more scratch than the library's static device array (no-alloc call)";
        default: return "unknown status";
    }
}

extern "C" int dflash_version(void) { return 100; }
