// The fixed-reference attention instances: launches of one range of work
// items (a dense call, or a single query group without key-range pieces),
// the block-sparse list mode, and launches of several ranges (query groups,
// key-range pieces). Same kernel template as attention.hip; this source is
// built with the VGPR form of the MFMA instructions, so the score
// accumulators of S^T = K Q^T live in VGPRs and the softmax reads them in
// place, while Q and O stay in AGPRs through their register-class hints. That
// removes the 32 accumulator-to-VGPR copies per half tile of keys the AGPR
// form needs (measured on the 58,758-key dense call: 60.6 -> 58.5 ms; on the
// streaming chunk's grouped call 2.03 -> 2.00 ms; the same bits). The
// online-softmax instances keep the AGPR form in attention.hip: their
// rescaling path needs the VGPRs.
#define H3_ATTN_SCORES_IN_VGPR 1
#include "h3_attention_kernel.h"

namespace h3 {

void launch_attention_fixed(bool sparse, dim3 grid, const AttnArgs &a, hipStream_t stream) {
    if (sparse)
        attention_fwd_kernel<true, true, false><<<grid, kThreads, 0, stream>>>(a);
    else
        attention_fwd_kernel<false, true, false><<<grid, kThreads, 0, stream>>>(a);
}

void launch_attention_fixed_multi(dim3 grid, const AttnArgs &a, hipStream_t stream) {
    attention_fwd_kernel<false, true, true><<<grid, kThreads, 0, stream>>>(a);
}

}  // namespace h3
