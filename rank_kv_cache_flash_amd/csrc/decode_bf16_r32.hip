// decode_bf16_r32.hip -- the split kernel of decode.hip for bf16 latent
// caches at rank 32 (H 64 and 128, every factor dtype), in a translation unit
// of its own so that it can be built with the machine scheduler's max-ILP
// strategy (build.py).  That order suits the short, latency-bound grids of
// this shape, e.g. one LLaVA-7B layer (1 sequence x 32 heads, 1088 tokens):
// 5.01 -> 4.87 us per launch on MI355X.  The rank-64 instance measured 0.5 %
// slower with the same strategy, so the other instances keep the default.
// The kernel and its launch helpers are those of decode.hip; only this
// unit's dispatch entry is compiled from it.
#define WSVD_DECODE_BF16_R32_UNIT 1
#include "decode.hip"
