// backward.hpp -- the backward's workspace layout, shared by its entry points and its kernels.
#pragma once

#include <stddef.h>

namespace gqa {

// The workspace holds two per-row float arrays, each padded to 64 floats (256 bytes): dout . out,
// then the forward's log-sum-exp times log2 e.
constexpr size_t backward_row_array_floats(size_t rows) { return (rows + 63) / 64 * 64; }

}  // namespace gqa
