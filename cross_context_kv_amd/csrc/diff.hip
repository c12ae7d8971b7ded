// Block-sparse diff encode / decode (a8, a9): not built yet.
#include "../../include/kvfix.h"

extern "C" size_t kvfix_diff_encode_workspace(int32_t, int32_t, int32_t, int32_t) { return 0; }
extern "C" kvfix_status kvfix_diff_encode(const kvfix_plane*, const kvfix_plane*, const kvfix_plane*,
                                          const kvfix_plane*, const kvfix_rope*, float,
                                          const kvfix_diff*, int32_t*, void*, size_t, void*) {
  return KVFIX_ERR_UNSUPPORTED;
}
extern "C" kvfix_status kvfix_diff_decode(const kvfix_plane*, const kvfix_plane*, const kvfix_diff*,
                                          const kvfix_rope*, const kvfix_plane*, const kvfix_plane*,
                                          void*) {
  return KVFIX_ERR_UNSUPPORTED;
}
