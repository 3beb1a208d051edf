// decode.hpp -- the decode entry for caches bounded to the sliding window, kept out of
// common.hpp so that the other kernels' sources (and the records taken on them) stay unchanged.
#pragma once

#include "common.hpp"

namespace gqa {

// Decode against caches bounded to the window (course page "Week 7. Attention", step 3): a.k,
// a.v hold a.Tkv = a.n_sink + a.window slots per sequence; entry e of a sequence sits in slot e
// (e < n_sink) or n_sink + (e - n_sink) mod window, and a.lens (required) counts every entry a
// sequence has had, unbounded by a.Tkv. Otherwise as launch_decode_bf16.
hipError_t launch_decode_window_cache_bf16(const DecodeArgs& a, hipStream_t s);

}  // namespace gqa
