// Host-side helpers shared by the C-ABI translation units (api.cpp and the
// allocation-free entry in noalloc.hip).  Not installed.
#pragma once

#include "../../include/moe_mi355x.h"

namespace moe {

// moe_forward_timed's body.  may_prepare = false refuses a layer whose
// binding is not prepared (preparing allocates) instead of preparing it.
moe_status forward_impl(const moe_layer *l, const moe_tensor *x, const moe_tensor *logits,
                        const moe_tensor *shared, moe_tensor *out, void *ws, size_t ws_bytes,
                        moe_routing_out *routing, void *stream, void *const *events,
                        bool may_prepare);

// Record `msg` as the calling thread's last error and return s.
moe_status set_error(moe_status s, const char *msg);

}  // namespace moe
