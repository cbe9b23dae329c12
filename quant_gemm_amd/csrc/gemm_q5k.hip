// Prefill GEMM for Q5_K weights (gfx950): the Q4_K kernel built with the
// Q5_K block layout (176 bytes, a high-bit plane between the header and the
// low nibbles) and the fifth bit merged into each int8 B operand.
#define MQ_Q5K 1
#include "gemm_q4k.hip"
