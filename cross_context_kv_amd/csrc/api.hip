// Status strings and version of the kvfix C ABI.
#include "../../include/kvfix.h"

extern "C" const char* kvfix_status_string(kvfix_status status) {
  switch (status) {
    case KVFIX_OK: return "KVFIX_OK";
    case KVFIX_ERR_ARG: return "KVFIX_ERR_ARG: invalid argument";
    case KVFIX_ERR_ALIGN: return "KVFIX_ERR_ALIGN: pointer or stride not 16-byte aligned";
    case KVFIX_ERR_CAPACITY: return "KVFIX_ERR_CAPACITY: diff or library buffer capacity exceeded";
    case KVFIX_ERR_HIP: return "KVFIX_ERR_HIP: HIP runtime or launch error";
    case KVFIX_ERR_UNSUPPORTED: return "KVFIX_ERR_UNSUPPORTED: dtype, head_dim or rank not compiled";
  }
  return "unknown kvfix status";
}

extern "C" int32_t kvfix_version(void) { return 100; }
