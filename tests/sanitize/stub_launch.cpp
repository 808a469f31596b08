// Stand-ins for the kernel launchers so that the host half of the C ABI
// (argument checks, plan, workspace sizing) links and runs without HIP. Any
// call that would launch returns an error instead; the driver never expects
// one to be reached with a valid plan.
#include <stdlib.h>

#include "../../gqa_attention_split_amd/csrc/mga_internal.h"

namespace mga {
int launch_partial(const Plan &, const void *, const void *, const void *, void *, void *, void *) { return 1; }
int launch_combine(const Plan &, void *, const void *, void *) { return 1; }
int launch_repack(const Plan &, const void *, void *, void *) { return 1; }
int scratch_ptr(void **) { return 1; }
// The chip size: MGA_TEST_CUS when set (to drive the split policy at other
// compute-unit counts), else the default.
int device_cus() {
    const char *e = getenv("MGA_TEST_CUS");
    return e && atoi(e) > 0 ? atoi(e) : kDefaultCUs;
}
}  // namespace mga
