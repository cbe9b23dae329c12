// Small-M configuration of the Q6_K prefill GEMM (gfx950).
//
// As for Q4_K: at a few dozen tokens the 128-token tiles are mostly empty.
// This instantiation of the same kernel source gives a workgroup 32 tokens
// x 128 weight rows, its four wavefronts side by side along the rows (32
// tokens x 32 rows each), and relies on split-K to fill the chip.
#define MQ_Q6K_TN 1
#define MQ_Q6K_WM 1
#define MQ_Q6K_WN 4
#define MQ_Q6K_SMALL 1
#include "gemm_q6k.hip"
