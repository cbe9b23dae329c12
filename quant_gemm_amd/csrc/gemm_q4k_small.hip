// Small-M configuration of the Q4_K prefill GEMM (gfx950).
//
// At a few to a few dozen tokens (a speculative-decoding verify batch, a
// short prompt) the 128-token tiles of the main configuration are mostly
// empty rows. This instantiation of the same kernel source gives a
// workgroup 32 tokens x 256 weight rows, its four wavefronts side by side
// along the rows (each 32 tokens x 64 rows, 1 x 2 MFMA tiles of 32 x 32),
// and relies on split-K to fill the chip. Everything else (staging, arithmetic, epilogue, split-K
// reduction) is the main kernel's.
#define MQ_Q4K_TM 1
#define MQ_Q4K_TN 2
#define MQ_Q4K_WM 1
#define MQ_Q4K_WN 4
#define MQ_Q4K_OCC 2
#define MQ_Q4K_SMALL 1
#include "gemm_q4k.hip"
