// Host-side settings of the per-launch device timing (ff_prof.h): which
// kernel families get event pairs.
#include "ff_prof.h"

namespace ff {

void dev_profiler_families(Profiler* p, unsigned families) {
  if (p) p->families = families;
}

}  // namespace ff
