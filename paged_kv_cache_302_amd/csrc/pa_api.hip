// ABI version and status strings of libpa.
#include "pa.h"

extern "C" int pa_abi_version(void) { return 8; }

extern "C" const char* pa_status_str(int status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_INVALID_ARG: return "invalid argument (null pointer, bad or inconsistent size)";
        case PA_ERR_UNSUPPORTED: return "unsupported configuration (head_size must be 64/128, block_size 16)";
        case PA_ERR_MISALIGNED: return "misaligned pointer or stride (16-byte alignment required)";
        case PA_ERR_LAUNCH: return "kernel launch failed";
        case PA_ERR_NO_SPACE: return "not enough free blocks, or an output buffer too small";
        case PA_ERR_SCRATCH_TOO_SMALL:
            return "the v2 partials exceed the fixed 48 MiB scratch of pa_decode_v2_noalloc";
        default: return "unknown status";
    }
}

