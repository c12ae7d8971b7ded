// Draft attention-mass score (a3): not built yet.
#include "../../include/kvfix.h"

extern "C" size_t kvfix_score_draft_workspace(int32_t, int32_t, int32_t, int32_t, int32_t, int32_t) {
  return 0;
}
extern "C" kvfix_status kvfix_score_draft(const void*, int32_t, int32_t, const kvfix_plane*, int32_t,
                                          const kvfix_rope*, float*, void*, size_t, void*) {
  return KVFIX_ERR_UNSUPPORTED;
}
