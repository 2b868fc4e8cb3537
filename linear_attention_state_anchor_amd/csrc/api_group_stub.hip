// placeholder until the group path lands
#include "sr_internal.hpp"
extern "C" {
size_t sr_packed_layer_bytes(int32_t, int32_t, int32_t, int32_t, int32_t) { return 0; }
int sr_pack_gdn_layer(const void*, const void*, const void*, int32_t, int32_t, int32_t,
                      int32_t, int32_t, void*, void*) { return SR_ESHAPE; }
size_t sr_replay_group_workspace_bytes(const sr_group_desc*) { return 0; }
int sr_replay_group(const sr_group_desc*, const sr_gdn_layer_weights*, const void*,
                    const int32_t*, float*, float*, void*, size_t, void*) { return SR_ESHAPE; }
}
