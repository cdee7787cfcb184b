// launch_stubs.cpp -- stand-ins for the kernel launchers, linked only into a
// host-only build of the C ABI's validation and planning code (the
// sanitizer test builds it with -fsanitize=address,undefined).  A
// validation test never reaches a launch, so every stand-in aborts.
#include <cstdlib>

#include "../../paged_top_indexer_amd/csrc/qsa_launch.h"

namespace qsa {

int launch_select(const SelectArgs&, const SelectPlan&, void*, bool) { std::abort(); }
int launch_paged_logits(const SelectArgs&, const SelectPlan&, void*) { std::abort(); }
int launch_topk_rows(const SelectArgs&, void*) { std::abort(); }
int launch_metadata(const MetaArgs&, void*) { std::abort(); }
int launch_attn(const AttnArgs&, const AttnPlan&, void*) { std::abort(); }
int static_scratch(void**) { std::abort(); }

}  // namespace qsa
