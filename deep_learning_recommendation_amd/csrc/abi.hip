// Library-wide entry points: version, status strings, last HIP error.
#include "common.hpp"

namespace dlrm {
thread_local int g_last_hip_error = 0;
}

extern "C" int dlrm_abi_version(void) { return DLRM_ABI_VERSION; }

extern "C" const char* dlrm_strerror(int status) {
  switch (status) {
    case DLRM_OK: return "ok";
    case DLRM_E_INVALID: return "invalid argument (null pointer, size, alignment or layout out of range)";
    case DLRM_E_WORKSPACE: return "workspace too small";
    case DLRM_E_HIP: return "HIP launch failed (see dlrm_last_hip_error)";
    case DLRM_E_UNSUPPORTED: return "valid but unsupported configuration";
    default: return "unknown status";
  }
}

extern "C" int dlrm_last_hip_error(void) { return dlrm::g_last_hip_error; }
