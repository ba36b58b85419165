// ring_state.h -- the device-side check of a request's ring state, shared by
// the kernels that read it (device code only).
//
// The state (ring_start, cache_len, next_pos) lives on the device and is
// updated by the kernels themselves, so the host cannot check it before a
// call.  It is usable when 0 <= ring_start < W, 0 <= cache_len <= W,
// next_pos >= 0, and next_pos + Tq (Tq = 1 for a decode step) stays within
// int32 ("Dense vs sliding-window sparse attention" blog, §3.2: a start index
// and a fill count over W slots; logical positions only grow).  (A ring that
// claims more rows than positions so far, cache_len > next_pos, is usable:
// its slots of negative positions are never visible.)  A
// request whose state is not usable writes nothing to its caches, its sink
// cache or its state; its attention sees no key (a decode step's output is
// zero).  This keeps every write of the step inside the caller's buffers
// whatever the state holds.
#pragma once

#include <limits.h>

namespace swa {

__device__ __forceinline__ bool ring_state_ok(int rs, int cl, int np, int W, int Tq) {
    return rs >= 0 && rs < W && cl >= 0 && cl <= W && np >= 0 && np <= INT_MAX - Tq;
}

}  // namespace swa
