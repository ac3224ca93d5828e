// Host-side interface used by the cascade (shared-prompt) decode.
#pragma once

#include "pa_internal.h"

namespace pa {

// Context split of the shared-prompt chunk of a cascade decode: few query rows per group over a
// long prompt make that chunk bandwidth-bound, so the split aims at one workgroup per CU (a second
// resident round gains nothing and every extra range adds merge traffic).
PrefillSplit prompt_split(int num_groups, int max_group_size, int num_kv_heads, int group,
                          int head_dim, int prefix_len);

}  // namespace pa
