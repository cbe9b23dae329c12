/*
 * mq.h - k-quant weight matmul on AMD MI355X (gfx950): the C ABI.
 *
 * The operation is the quantized matmul of the CUDA prefill/decode path of
 * the minfer pages: GGML Q4_K / Q5_K / Q6_K weight super-blocks multiplied against
 * f32 activations that are first quantized to a per-32 int8 plane
 * (minfer Features, "GPU — CUDA": int8 MMQ GEMMs for q4_K and q6_K fed by an
 * int8 activation plane; decode by the MMVQ weight-streaming path.
 * minfer Compute Graph Design, §9.3 Execution dispatch: the activation is
 * quantized once and that plane serves every matmul that reads it.)
 *
 * Conventions for every entry point
 *   - Pointers are device pointers owned by the caller. The calls enqueue
 *     kernels on `stream` (a hipStream_t passed as void*, NULL = the null
 *     stream) and return; nothing synchronizes. Inputs are read-only; outputs
 *     are overwritten. The library never allocates or frees device memory
 *     and keeps no buffers between calls: the buffers belong to the caller,
 *     as they belong to the allocator and not to the kernels on the pages
 *     (minfer Compute Graph Design, §1.4 Core invariants).
 *   - Workspace. Three plans use scratch memory: a GEMM with too few output
 *     tiles to fill the device splits K into nsplit [M][N] f32 planes of
 *     partial sums (added in a fixed order, so results do not depend on
 *     scheduling); a Q6_K GEMM of at least 512 tokens (on matrices of at
 *     most 2^28 weights) first expands W into the limb planes of
 *     mq_expand_q6k there, decoding each block once per call instead of
 *     once per token tile, with the same result bit for bit; and the fused
 *     FFN's two-pass form keeps g and u. The
 *     *_ws entry points take that memory from the caller (ws, ws_bytes);
 *     mq_matmul_workspace / mq_ffn_q4k_workspace give the bytes a call
 *     with the same arguments needs (0 when its plan uses none). ws == NULL
 *     (with ws_bytes == 0) selects the workspace-free plan: GEMMs never
 *     split K, and the FFN runs its one-launch GEMM. A non-NULL ws must be
 *     16-byte aligned and hold at least the bytes the query gives, else the
 *     call fails with MQ_ERR_WORKSPACE and launches nothing; the one
 *     exception is a Q6_K GEMM that would expand W, which with at least
 *     the split-K part (the query's figure less the planes) runs on the raw
 *     blocks instead, with the same result. The entry
 *     points without a ws argument take the workspace-free plan. The
 *     workspace is read and written only by the kernels of the call that
 *     receives it: calls in flight at the same time need distinct
 *     workspaces (calls in order on one stream may share one).
 *   - Arguments are validated on the host before any HIP call. A failed
 *     check returns a nonzero mq_status and nothing is launched; the
 *     calling thread's mq_last_error() then names the argument and its value.
 *     Errors are never turned into a silent fallback (minfer Compute Graph
 *     Design, §7.4 Error contract).
 *   - After the checks the current device must be gfx950 (queried at run
 *     time, minfer Architecture, §5.3 GPU safety), else MQ_ERR_UNSUPPORTED.
 *   - Sizes are element counts. K must be a positive multiple of 256 (one
 *     super-block) up to 2^31-1; M and N may be any positive value up to
 *     0x7fff0000 (2^31 - 65536).
 *   - There is no device-side validation of data. Non-finite activations are
 *     a precondition violation with unspecified output.
 *   - Calls are thread-safe. Calls that overlap in time on the same output
 *     buffers race, as for any kernel.
 *
 * Data layout in device memory
 *   x    f32  [M][ldx]   activations, token-major (row t = one token)
 *   q    int8 [M][K]     quantized activations, token-major
 *   d    f32  [M][K/32]  per-block activation scale
 *   s    f32  [M][K/32]  per-block d * (sum of the block's q)
 *   W    N rows, each K/256 consecutive super-blocks, rows back to back:
 *          Q4_K: 144-byte blocks  (f16 d, f16 dmin, 12 B of 6-bit scale and
 *                min codes, 128 B of 4-bit quants); row = K/256*144 bytes
 *          Q5_K: 176-byte blocks  (f16 d, f16 dmin, the 12 B of codes of
 *                Q4_K, 32 B of fifth bits, 128 B of low nibbles); row =
 *                K/256*176 bytes
 *          Q6_K: 210-byte blocks  (128 B low nibbles, 64 B high bit pairs,
 *                16 int8 scales, f16 d); row = K/256*210 bytes
 *        (GGML's layouts: minfer Architecture, §6 Quantization & Tensor
 *        Layout; weights are [out][in] row-major, §4.5 Core invariants.)
 *   out  f32  [M][N]     token-major output (minfer Compute Graph Design,
 *                        §7.1: activations and outputs are token-major)
 *
 * Alignment: q, d and s must be 16-byte aligned; x and out 4-byte aligned.
 * W: 16-byte aligned for Q4_K and Q5_K, whose block fields are read as
 * 16-byte pieces (their rows are multiples of 16 bytes, so every row of an
 * aligned matrix is aligned too); 4-byte aligned for Q6_K, whose 210-byte
 * blocks fall on 2-byte boundaries within a row anyway and are read
 * through aligned dwords (so a slice from any even-length row offset is
 * accepted).
 */
#ifndef MQ_H
#define MQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MQ_ABI_VERSION 6

typedef enum {
    MQ_OK = 0,
    MQ_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, unknown path */
    MQ_ERR_SHAPE = 2,       /* K not a positive multiple of 256, ldx < K, too large */
    MQ_ERR_ALIGN = 3,       /* a pointer is not aligned as required */
    MQ_ERR_UNSUPPORTED = 4, /* the current device is not gfx950 */
    MQ_ERR_DEVICE = 5,      /* a HIP runtime query failed */
    MQ_ERR_LAUNCH = 6,      /* the kernel launch failed */
    MQ_ERR_WORKSPACE = 7    /* the workspace is smaller than the call needs */
} mq_status;

/* Weight formats, for mq_matmul_workspace. */
enum { MQ_FMT_Q4K = 0, MQ_FMT_Q5K = 1, MQ_FMT_Q6K = 2 };

/* Kernel path selectors for the *_ex entry points. */
enum { MQ_PATH_AUTO = 0, MQ_PATH_GEMV = 1, MQ_PATH_GEMM = 2 };

/*
 * Per-32 int8 activation quantization.
 * For each token t and block b of 32 consecutive values x[t][32b .. 32b+31]:
 *   amax = max |x|;  d[t][b] = amax / 127 (IEEE f32 division);
 *   q[t][32b+i] = d[t][b] == 0 ? 0 : clamp(roundf(x[t][32b+i] / d[t][b]), -127, 127)
 *                 (roundf rounds halves away from zero; d == 0 when amax == 0
 *                 or when amax / 127 underflows);
 *   s[t][b] = d[t][b] * (float)(sum_i q[t][32b+i]).
 * The pages require an on-the-fly activation quantization with per-subblock
 * sums (minfer Support Matrix, "Supported Quantization Formats") but do not
 * give the rounding rule; this is the reading taken, and the result is
 * bit-exact against it. x has row stride ldx >= K (elements).
 * Outputs q [M][K], d and s [M][K/32] are written in full.
 */
int mq_quantize_act(const float *x, int64_t M, int64_t K, int64_t ldx,
                    int8_t *q, float *d, float *s, void *stream);

/*
 * Producer-fused quantization, RMSNorm: the int8 plane of
 *   y[t][k] = (x[t][k] * r_t) * w[k],  r_t = f32(1 / sqrt(ss_t / K + eps)),
 * where ss_t = sum_k x[t][k]^2 is the exact sum rounded once to f64 and
 * 1 / sqrt(ss / K + eps) is evaluated with correctly rounded f64 operations;
 * the two products are f32 (no fused multiply-add). q, d and s are what
 * mq_quantize_act would write for y, so the matmuls take them unchanged.
 * The pages have the norm emit the int8 plane directly instead of an f32
 * tensor (minfer Features, "GPU — CUDA"); the op is RmsNorm{eps} with its
 * weight (minfer Compute Graph Design, "The Op vocabulary"). The arithmetic
 * is the reading taken: the pages give none.
 *   x  f32 [M][ldx] (16-byte aligned, ldx >= K and a multiple of 4)
 *   w  f32 [K] (16-byte aligned); eps finite and >= 0
 *   y  optional f32 [M][K] (16-byte aligned): when not NULL, y itself is
 *      written too.
 */
int mq_rmsnorm_quantize(const float *x, const float *w, int64_t M, int64_t K,
                        int64_t ldx, float eps, int8_t *q, float *d, float *s,
                        float *y, void *stream);

/*
 * Producer-fused quantization, SwiGLU: the int8 plane of
 *   y[t][k] = f32(g / (1 + exp(-g)))  * u[t][k],  g = g[t][k],
 * the SiLU evaluated in f64 (exp within an f64 ulp) and rounded once, the
 * product in f32. The op is SwiGLU = Silu(gate) * up (minfer Compute Graph
 * Design, "The Op vocabulary"), emitting the plane directly as the norm
 * above. g and u have row strides ldg and ldu, so the two halves of a
 * concatenated gate|up output ([M][2K], u = g + K, ldg = ldu = 2K) are read
 * in place.
 *   g, u  f32, 16-byte aligned, ldg and ldu >= K and multiples of 4
 *   y     optional f32 [M][K] (16-byte aligned), written when not NULL.
 */
int mq_swiglu_quantize(const float *g, const float *u, int64_t M, int64_t K,
                       int64_t ldg, int64_t ldu, int8_t *q, float *d, float *s,
                       float *y, void *stream);

/*
 * Q4_K matmul: out[t][n] = sum_k w[n][k] * d[t][k/32] * q[t][k], where
 * w[n][k] = d_blk * sc_j * q4 - dmin_blk * m_j for the weight's super-block
 * and 32-value sub-block j. The int8 dot of each 32-value sub-block is exact
 * (int32); scales, mins and the min term (which uses s) are applied in f32.
 * Result within 1e-4 * max|out| of the exact value for the workloads tested.
 * Small M runs the weight-streaming GEMV, larger M the int8 MFMA GEMM (the
 * CUDA dispatch splits decode from prefill by token count: minfer Support
 * Matrix, "CUDA notes"). MQ_PATH_AUTO switches at crossovers measured on
 * MI355X (GPU time per call): Q4_K runs the GEMV for M <= 2; up to 8 tokens
 * where its persistent stream takes them (rows of K <= 10752 and a plane of
 * at most 32 KB, 40 KB above 4 tokens) while M*N*K <= 4.2e8; otherwise up
 * to 16 tokens while M*N*K <= 2.6e8. Q5_K likewise (rows of K <= 6144;
 * 5.5e8 and 3.3e8). Q6_K
 * runs it for M <= 4, and up to 8 tokens where its LDS ring kernel takes the
 * plane while M*N*K <= 5.5e8. The GEMM uses 32-token tiles up to M = 64
 * (Q4_K, Q5_K) / 32 (Q6_K) and 128-token tiles above. The GEMV serves up to
 * mq_gemv_max_m() tokens when forced.
 * W as described above; q, d, s from mq_quantize_act (s is required).
 * Workspace-free plan: the GEMM never splits K (mq_matmul_q4k_ws, given a
 * workspace, may).
 */
int mq_matmul_q4k(const void *W, const int8_t *q, const float *d,
                  const float *s, int64_t M, int64_t N, int64_t K,
                  float *out, void *stream);

/*
 * Q6_K matmul: as mq_matmul_q4k with w[n][k] = d_blk * scales[j] * (q6 - 32)
 * for the weight's 16-value group j. s is not used and may be NULL.
 */
int mq_matmul_q6k(const void *W, const int8_t *q, const float *d,
                  const float *s, int64_t M, int64_t N, int64_t K,
                  float *out, void *stream);

/*
 * Q5_K matmul: as mq_matmul_q4k with 5-bit quants,
 * w[n][k] = d_blk * sc_j * q5 - dmin_blk * m_j, where q5 of position i of
 * sub-block j = 2c + h is the nibble (qs[32c + i] >> 4h) & 15 plus 16 times
 * bit j of qh[i] (q5_K is among the k-quants of the pages' decode path:
 * minfer Support Matrix, "Supported Quantization Formats"; GGML's block).
 * s is required. MQ_PATH_AUTO uses the Q4_K crossovers.
 */
int mq_matmul_q5k(const void *W, const int8_t *q, const float *d,
                  const float *s, int64_t M, int64_t N, int64_t K,
                  float *out, void *stream);

/*
 * As mq_matmul_q4k / mq_matmul_q5k / mq_matmul_q6k with the kernel chosen by `path`
 * (MQ_PATH_AUTO, MQ_PATH_GEMV, MQ_PATH_GEMM). MQ_PATH_GEMV requires
 * M <= mq_gemv_max_m() (M <= 8 for mq_ffn_q4k_ex). Both paths meet the same contract; tests use this
 * to check each path on the same inputs. Workspace-free plan.
 */
int mq_matmul_q4k_ex(const void *W, const int8_t *q, const float *d,
                     const float *s, int64_t M, int64_t N, int64_t K,
                     float *out, void *stream, int path);
int mq_matmul_q5k_ex(const void *W, const int8_t *q, const float *d,
                     const float *s, int64_t M, int64_t N, int64_t K,
                     float *out, void *stream, int path);
int mq_matmul_q6k_ex(const void *W, const int8_t *q, const float *d,
                     const float *s, int64_t M, int64_t N, int64_t K,
                     float *out, void *stream, int path);

/*
 * The matmuls with a caller workspace (see the conventions above): the
 * same result and contract, and the full plan, which may split K over the
 * workspace when the output has too few tiles to fill the device.
 * mq_matmul_workspace writes to *bytes the workspace a matmul of format fmt
 * (MQ_FMT_Q4K / Q5K / Q6K) with these M, N, K and path needs: nsplit * M *
 * N * 4 (0 when the plan splits nothing), plus, for a Q6_K GEMM that
 * expands W (M >= MQ_Q6K_EXPAND_MIN_M on a matrix of at most
 * MQ_Q6K_EXPAND_MAX_WEIGHTS weights), its planes: 2 * N * K + 4 * N * K /
 * 256 bytes (each part rounded up to 256). It validates M, N, K and path as
 * the matmul does. Measured on MI355X (3584 x 18944; the expansion itself
 * 42 us): the expansion plan takes 206 / 264 / 328 us at M = 512 / 768 /
 * 1024 against 227 / 298 / 393 us on the raw blocks, and breaks even near
 * M = 384.
 */
#define MQ_Q6K_EXPAND_MIN_M 512
#define MQ_Q6K_EXPAND_MAX_WEIGHTS (1ll << 28)
int mq_matmul_workspace(int fmt, int64_t M, int64_t N, int64_t K, int path,
                        int64_t *bytes);
int mq_matmul_q4k_ws(const void *W, const int8_t *q, const float *d,
                     const float *s, int64_t M, int64_t N, int64_t K,
                     float *out, void *ws, int64_t ws_bytes, void *stream,
                     int path);
int mq_matmul_q5k_ws(const void *W, const int8_t *q, const float *d,
                     const float *s, int64_t M, int64_t N, int64_t K,
                     float *out, void *ws, int64_t ws_bytes, void *stream,
                     int path);
int mq_matmul_q6k_ws(const void *W, const int8_t *q, const float *d,
                     const float *s, int64_t M, int64_t N, int64_t K,
                     float *out, void *ws, int64_t ws_bytes, void *stream,
                     int path);

/*
 * Fused FFN up half: the gate and up projections and SwiGLU in one call,
 * producing the int8 plane of the down projection's input. The pages fuse
 * the decode FFN as one gate|up matmul with an in-place SwiGLU (FusedFFN,
 * minfer Compute Graph Design, "The Op vocabulary") and have the SwiGLU
 * epilogue emit the int8 plane (minfer Features, "GPU — CUDA").
 *   g = the Q4_K matmul of Wg with the plane (q, d, s), u the same with Wu,
 *       each as mq_matmul_q4k computes it (f32, within its tolerance);
 *   y[t][n] = f32(SiLU(g[t][n]) in f64) * u[t][n], as mq_swiglu_quantize;
 *   qo [M][N], do_ and so [M][N/32]: the quantizer's plane of y (exactly
 *       what mq_quantize_act would write for y);
 *   y  optional f32 [M][N], written when not NULL.
 * Wg and Wu are N rows of K each (Q4_K layout); N is a positive multiple of
 * 256 (it is the down projection's K).
 * Plans. mq_ffn_q4k_ws with a workspace: up to 128 tokens in two passes,
 * g and u into the workspace (2*M*N f32, followed by the split-K planes of
 * the GEMMs when they split), then the SwiGLU quantizer. The first pass is
 * the GEMV up to 8 tokens under MQ_PATH_AUTO (both matrices as one
 * persistent stream where the plane fits it) and the GEMMs above;
 * MQ_PATH_GEMV forces the GEMV (M <= 8), MQ_PATH_GEMM the GEMMs. Above 128
 * tokens, and at every M without a workspace (mq_ffn_q4k, mq_ffn_q4k_ex,
 * or ws == NULL), one GEMM launch does it all: its tiles pair 64 gate rows
 * with the same 64 up rows and apply SwiGLU and the quantizer in their
 * epilogue. MQ_PATH_GEMV without a workspace is MQ_ERR_WORKSPACE.
 * mq_ffn_q4k_workspace gives the bytes of the two-pass form (0 where the
 * one-launch GEMM runs); it validates M, N, K and path as the call does.
 * Alignment as for the matmuls; qo, do_, so and y 16-byte aligned.
 */
int mq_ffn_q4k(const void *Wg, const void *Wu, const int8_t *q, const float *d,
               const float *s, int64_t M, int64_t N, int64_t K, int8_t *qo,
               float *do_, float *so, float *y, void *stream);
int mq_ffn_q4k_ex(const void *Wg, const void *Wu, const int8_t *q, const float *d,
                  const float *s, int64_t M, int64_t N, int64_t K, int8_t *qo,
                  float *do_, float *so, float *y, void *stream, int path);
int mq_ffn_q4k_workspace(int64_t M, int64_t N, int64_t K, int path, int64_t *bytes);
int mq_ffn_q4k_ws(const void *Wg, const void *Wu, const int8_t *q, const float *d,
                  const float *s, int64_t M, int64_t N, int64_t K, int8_t *qo,
                  float *do_, float *so, float *y, void *ws, int64_t ws_bytes,
                  void *stream, int path);

/*
 * Registration-time weight planes for the prefill GEMM. The pages build
 * weight-expansion planes for q6_K and a decoded-scale plane for q4_K when
 * weights are registered, and their MMQ GEMM reads those instead of
 * decoding the raw blocks per tile (minfer Features, "GPU — CUDA": W_exp /
 * W_dsc, about 3.3 GB for about +6% prefill). Build once per weight matrix;
 * the planes are plain device arrays owned by the caller. They serve the
 * GEMM (prefill) only: a decode step reads the raw blocks (mq_matmul_*),
 * which are 2.4x (Q6_K) fewer bytes.
 *
 * mq_expand_q6k: W (Q6_K, N rows of K) -> lo, hi int8 [N][K] and dw f32
 * [N][K/256]: for every weight p = sc_g * (q - 32) (g its 16-value group,
 * p in -4064..4096) is lo + 64 * hi with lo in 0..63, hi in -64..64; dw is
 * each super-block's d. Exact. W 4-byte aligned; lo, hi, dw 16-byte
 * aligned.
 */
int mq_expand_q6k(const void *W, int64_t N, int64_t K, int8_t *lo, int8_t *hi,
                  float *dw, void *stream);

/*
 * Q6_K matmul from the expansion planes: the same result and contract as
 * mq_matmul_q6k on the blocks they were built from (f32, within its
 * tolerance), always on the int8 MFMA GEMM (32-token tiles up to M = 32).
 * lo, hi 16-byte aligned, dw 4-byte aligned; q, d, out as for the matmuls.
 * ws / ws_bytes as for mq_matmul_q6k_ws with MQ_PATH_GEMM (the same split
 * of K; NULL = no split).
 */
int mq_matmul_q6k_x(const int8_t *lo, const int8_t *hi, const float *dw,
                    const int8_t *q, const float *d, int64_t M, int64_t N,
                    int64_t K, float *out, void *ws, int64_t ws_bytes,
                    void *stream);

/*
 * mq_dsc_q4k: W (Q4_K, N rows of K) -> fw, fm f32 [N][K/32] with
 * fw = d * sc_j and fm = dmin * m_j for each 32-value sub-block j (exact:
 * an f16 times a 6-bit code). W, fw, fm 16-byte aligned.
 */
int mq_dsc_q4k(const void *W, int64_t N, int64_t K, float *fw, float *fm,
               void *stream);

/*
 * Q4_K matmul reading the quants from W and the factors from the
 * decoded-scale planes (no block header decoded per tile): the same result
 * and contract as mq_matmul_q4k, always on the GEMM (32-token tiles up to
 * M = 64). fw, fm as built by mq_dsc_q4k from this W; s is required.
 * ws / ws_bytes as for mq_matmul_q4k_ws with MQ_PATH_GEMM.
 */
int mq_matmul_q4k_dsc(const void *W, const float *fw, const float *fm,
                      const int8_t *q, const float *d, const float *s,
                      int64_t M, int64_t N, int64_t K, float *out, void *ws,
                      int64_t ws_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the Q6_K
 * matmul of mq_matmul_q6k_ws (MQ_PATH_AUTO) with its split-K partial sums
 * kept in a static device array of the library instead of a caller
 * workspace; it never takes the expansion plan, so it needs nsplit * M * N
 * * 4 bytes (mq_matmul_workspace's figure without the planes) and gives the
 * same result. The array holds MQ_STATIC_SCRATCH_BYTES (32 MiB); each
 * GPU the library runs on holds its own copy until the process ends, and its
 * address is looked up once per device on the first call there that needs
 * it. A call whose split-K plan needs more (e.g. 3314 x 3584 x 18944 needs
 * about 95 MB) fails with MQ_ERR_WORKSPACE before anything is launched. The call
 * allocates nothing. All calls on one GPU share its array, which keeps the
 * last call's partial sums (every call overwrites what it reads): calls
 * that overlap in time on one GPU, on any streams, race and give wrong
 * results. Same arguments, result and alignment rules as mq_matmul_q6k.
 */
#define MQ_STATIC_SCRATCH_BYTES (32u << 20)
int mq_matmul_q6k_static(const void *W, const int8_t *q, const float *d,
                         const float *s, int64_t M, int64_t N, int64_t K,
                         float *out, void *stream);

/*
 * Measurement hook. The next matmul or quantizer call of the calling thread
 * (mq_matmul_*, mq_ffn_q4k*, mq_quantize_act) launches its main kernel with
 * hipExtLaunchKernel, which records start_event and stop_event (hipEvent_t,
 * created by the caller; either may be NULL) at that kernel's own dispatch
 * start and end, so
 * hipEventElapsedTime gives the kernel's duration without the launch gap an
 * event recorded before the call would include. A split-K GEMM's reduction
 * kernel is not covered. The request is consumed by that call, and dropped
 * by any other mq_* call in between that launches kernels (the workspace
 * queries leave it). Always returns MQ_OK.
 */
int mq_time_next_kernel(void *start_event, void *stop_event);

/* Largest M the GEMV path serves (MQ_PATH_GEMV); 16. */
int64_t mq_gemv_max_m(void);

/* Message for the calling thread's last failed call ("" if none). The
 * pointer stays valid until the thread's next mq_* call. */
const char *mq_last_error(void);

/* MQ_ABI_VERSION of the loaded library. */
int mq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MQ_H */
