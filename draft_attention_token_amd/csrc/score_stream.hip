// Token importance, single-pass streaming form (K read once): not built yet.
#include "score_common.h"

namespace sp {

bool score_stream_supported(const AttnShape &, int, int) { return false; }

size_t score_stream_ws(const AttnShape &, int, int) { return 0; }

hipError_t launch_score_stream(const AttnShape &, const SegTable &, int, const void *,
                               const void *, float *, void *, size_t, hipStream_t,
                               bool *supported) {
  *supported = false;
  return hipSuccess;
}

}  // namespace sp
