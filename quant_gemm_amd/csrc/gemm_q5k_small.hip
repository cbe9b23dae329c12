// Small-M configuration of the Q5_K prefill GEMM (gfx950): 32 tokens x 128
// weight rows per workgroup, four wavefronts side by side along the rows
// (32 x 32 each), split-K to fill the chip.
#define MQ_Q5K 1
#define MQ_Q4K_TM 1
#define MQ_Q4K_TN 1
#define MQ_Q4K_WM 1
#define MQ_Q4K_WN 4
#define MQ_Q4K_OCC 2
#define MQ_Q4K_SMALL 1
#include "gemm_q4k.hip"
