// Library-wide entry points: status names and ABI version.
#include "common.h"

extern "C" const char *eagle3_status_string(int status) {
    switch (status) {
        case EAGLE3_OK: return "EAGLE3_OK";
        case EAGLE3_ERR_ARG: return "EAGLE3_ERR_ARG: null pointer, negative size or misaligned tensor";
        case EAGLE3_ERR_UNSUPPORTED: return "EAGLE3_ERR_UNSUPPORTED: shape or option not handled by this library";
        case EAGLE3_ERR_TREE: return "EAGLE3_ERR_TREE: parent[] is not a rooted tree in topological order";
        case EAGLE3_ERR_RANGE: return "EAGLE3_ERR_RANGE: id out of range";
        case EAGLE3_ERR_HIP: return "EAGLE3_ERR_HIP: kernel launch failed";
        case EAGLE3_ERR_WORKSPACE: return "EAGLE3_ERR_WORKSPACE: workspace too small";
        default: return "EAGLE3: unknown status";
    }
}

extern "C" int eagle3_abi_version(void) { return 3; }
