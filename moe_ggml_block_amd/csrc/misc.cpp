// Library identification and status strings (host only).
#include "qmv.h"

extern "C" const char *qmv_version(void) { return "qmv 0.1.0 gfx950"; }

extern "C" const char *qmv_strerror(int status) {
    switch (status) {
        case QMV_OK: return "ok";
        case QMV_EINVAL: return "invalid argument (shape, block multiple, topk, null pointer or workspace size)";
        case QMV_EALIGN: return "pointer alignment requirement not met";
        case QMV_ELAUNCH: return "HIP kernel launch failed";
        case QMV_EUNSUPPORTED: return "shape outside what this build implements";
        default: return "unknown status";
    }
}
