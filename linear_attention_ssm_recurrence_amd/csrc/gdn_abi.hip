// Library-wide C-ABI entry points: error text and ABI version.
#include "gdn.h"

extern "C" const char* gdn_strerror(int code) {
  switch (code) {
    case GDN_OK: return "success";
    case GDN_ENULL: return "a required pointer is NULL";
    case GDN_ESIZE: return "a size is non-positive, too large, or inconsistent with another";
    case GDN_EUNSUPPORTED: return "shape not supported by the library";
    case GDN_EALIGN: return "a float4-accessed pointer is not 16-byte aligned";
    case GDN_ELAUNCH: return "the HIP runtime rejected a kernel launch";
  }
  return "unknown gdn error code";
}

extern "C" int gdn_abi_version(void) { return 1; }
