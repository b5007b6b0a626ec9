// Internal declarations shared by the host-side sources of libh3block.
// Nothing here is part of the public ABI (include/h3block.h).
#pragma once

#include <cstddef>
#include <cstdint>

#include "h3block.h"

namespace h3 {

constexpr int64_t kHeadDim = 128;
constexpr int64_t kMaxHidden = 16384;
constexpr size_t kWsAlign = 256;

// Byte offsets and row strides of the block's workspace buffers.
struct WsLayout {
    int64_t off[H3_WS_COUNT];
    int64_t ld[H3_WS_COUNT];
    int64_t cols[H3_WS_COUNT];
    size_t total;
};
bool ws_layout(const h3_dims *d, int64_t L_buf, WsLayout *out);

// Validation of dims shared by several checks.
int check_dims(const h3_dims *d);

}  // namespace h3
