// Internal declarations of the two-level (group) path of libepget.  Not
// part of the public ABI (that is include/ep_get.h).
#pragma once

#include "ep_internal.h"

namespace epget {

// Two-level (group) path: G groups of ranks_per_group ranks, rank slices of
// S rows, group slices of SG rows (group_rows = G * SG).
struct HierParams {
    int32_t G, ranks_per_group, S, SG;
    int64_t group_rows;
};

// status (may be null): lowered to EP_ERR_CAPACITY when a group has more
// tokens than SG rows.
hipError_t launch_group_layout(int32_t T, int32_t R, const HierParams &h, const uint8_t *map,
                               int32_t *group_slot, int32_t *status, hipStream_t stream);
// Stage-1 dispatch: each token's row to its group rows.
hipError_t launch_group_dispatch(const CopyParams &c, const HierParams &h, const uint16_t *x,
                                 const int32_t *group_slot, uint16_t *group_buf, hipStream_t stream);
// Stage-2 dispatch: each group row to the entries of that group.
hipError_t launch_expand(const CopyParams &c, const HierParams &h, const DispatchArgs &a,
                         const int32_t *group_slot, const uint16_t *group_buf, hipStream_t stream);
// Stage-1 combine: per-(token, group) partial sums into the group rows.
hipError_t launch_combine_partial(const CopyParams &c, const HierParams &h, const uint16_t *y,
                                  const int32_t *slot, const float *w, const int32_t *group_slot,
                                  uint16_t *group_buf, hipStream_t stream);
// Stage-2 combine: the sum of a token's group rows.
hipError_t launch_combine_groups(const CopyParams &c, const HierParams &h, const uint16_t *group_buf,
                                 const int32_t *group_slot, uint16_t *out, hipStream_t stream);

}  // namespace epget
