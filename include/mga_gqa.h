/*
 * mga_gqa.h -- C ABI of the MI355X (gfx950) fused GQA exp-sum-div library.
 *
 * Operation (Mirage documentation, GQA tutorial, "Mirage: Define GQA
 * Computation Graph"; the same graph is section 1 of the kaispace blog post
 * on Mirage's muGraph search):
 *
 *     A = Q K,  E = exp(A),  S = rowsum(E) over the keys,  O = (E / S) V
 *
 * with no 1/sqrt(d) scale and no max subtraction. Per (b, i) row:
 *     O[b,i,j] = sum_n exp(a_n) V[b,n,j] / sum_n exp(a_n),
 *     a_n      = sum_d Q[b,i,d] K[b,d,n].
 *
 * The library evaluates it as split-KV partial sums plus a combine, the
 * two-block-graph form that the blog's sections 2.1 and 4.2-4.3 describe for
 * the "attention" search configuration (a for-loop over the key dimension with
 * accumulation, then a combine across grid blocks). Because the graph
 * subtracts no running maximum, partials combine by plain sums:
 *     O = (sum_s L_s o_s) / (sum_s L_s),  o_s = W_s / L_s,
 *     W_s = sum_{n in split s} e_n V[n],  L_s = sum_{n in split s} e_n.
 *
 * Data layout (IEEE fp16, device memory). The default entry points take
 * row-major contiguous tensors, the graph inputs' default strides (kaispace
 * blog, section 2: new_input records a shape and strides, row-major unless
 * given, and compile() requires run-time tensors to match them):
 *     q [B][M][D]      query rows (axis 0 = batch x KV heads)
 *     k [B][D][N]      keys stored head-dim-major ("pre-transposed")
 *     v [B][N][D]      values
 *     o [B][M][D]      output, written with round-to-nearest-even
 * mga_gqa_forward_strided takes the same logical tensors as strided views
 * instead (see there), including K stored key-major.
 * The head dimension D is 64 (the tutorial graph) or 128 (the tutorial's
 * launch example: Q (64, 1, 128), K (64, 128, 4096), V (64, 4096, 128)).
 * Pointers must be 16-byte aligned. N is at most 2^30 / D - 1 and need not
 * be a multiple of anything: contiguous K whose rows (N keys) do not start
 * on 16-byte boundaries (N % 8 != 0) is first copied by the library into the
 * workspace with rows of ceil8(N) keys (one extra pass over K).
 *
 * Numerics: fp16 MFMA products with fp32 accumulation; E = exp(A) in fp32
 * via the hardware exp2 of log2(e) Q rounded to fp16; P = fp16(E), rounded to
 * nearest even, is the tensor E of the fp16 graph: it feeds the second
 * product and its fp32 row-sum is S, so numerator and denominator use the
 * same weights. With more than one split each partial o_s is stored rounded
 * to fp16 (L_s stays fp32), which adds at most 2^-11 max_s |o_s| to the
 * error. Results are deterministic for a fixed (shape, splits): every
 * sum runs in a fixed order and no atomics are used. Inputs whose scores reach
 * ln(65504) ~ 11.09 overflow fp16 P; results are then undefined (the graph
 * itself overflows there). At the other end, a score below ln(2^-24) ~ -16.6
 * gives P = 0 (fp16 flushes it): a row all of whose scores lie there has
 * S = 0 and its output is 0/0 = NaN, as in the fp16 graph (the exact
 * real-valued softmax would still be finite). Scores between -16.6 and
 * ln(2^-14) ~ -9.7 land on fp16 subnormals.
 *
 * Ownership and asynchrony: the caller owns q, k, v, o and the workspace; the
 * library allocates and frees nothing on the device and keeps no device state,
 * so calls are reentrant. Work is enqueued on `stream` (a hipStream_t; NULL =
 * the legacy default stream) with no host synchronisation; a fault inside a
 * kernel surfaces at the caller's next synchronisation.
 *
 * Errors: every entry point validates its arguments on the host before any
 * launch and returns an mga_status; on a nonzero status nothing was launched,
 * except MGA_ERR_HIP, which reports a launch the runtime refused: the status
 * hipLaunchKernel returned for that launch, not an error that an earlier HIP
 * call of the caller left for hipGetLastError.
 */
#ifndef MGA_GQA_H
#define MGA_GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. The numbering follows the transpiler error codes the kaispace
 * blog lists in its section 5.1 (success 0, insufficient shared memory 1,
 * layout error 2, config error 3), extended for this library. */
typedef enum {
    MGA_OK = 0,
    MGA_ERR_INVALID_VALUE = 1, /* null pointer, B or M < 0, N < 1, splits < 0      */
    MGA_ERR_LAYOUT = 2,        /* pointer not 16-byte aligned, or a stride the
                                  strided entry point does not take                 */
    MGA_ERR_CONFIG = 3,        /* D not 64/128, splits > ceil(N / 128), N > 2^30/D - 1,
                                  grid too big                                      */
    MGA_ERR_WORKSPACE = 4,     /* workspace missing, misaligned or too small        */
    MGA_ERR_HIP = 5,           /* a kernel launch failed                            */
    MGA_ERR_SCRATCH = 6        /* mga_gqa_forward_noalloc: workspace above its scratch */
} mga_status;

/* Keys per pipeline stage; split chunks are whole multiples of it. */
#define MGA_KEY_BLOCK 128
/* Head dimensions supported by this build. */
#define MGA_HEAD_DIM 64
#define MGA_HEAD_DIM_WIDE 128

/* Human-readable text for a status code (static storage, never NULL). The
 * codes follow the transpiler error codes of the kaispace blog, section 5.1
 * (success 0, insufficient shared memory 1, layout error 2, config error 3). */
const char *mga_status_string(int status);

/* Chip size. The split policy fills the compute units of the calling
 * thread's current HIP device: the planning calls (this one, and every call
 * that sizes a workspace, plans or validates) ask the runtime once per device
 * for its compute-unit count (hipDeviceAttributeMultiprocessorCount: 256 on
 * MI355X in its default single-partition mode) and assume 256 when no device
 * answers, e.g. on a host without a GPU. Beyond that query they make no HIP
 * call, launch nothing and allocate nothing. Plan, size and launch with the
 * same device current: split counts and workspace sizes can differ between
 * devices of different sizes.
 *
 * Split policy (host only, deterministic for a given chip size): the number
 * of KV splits the library uses for this shape when the caller passes
 * splits = 0. Always in
 * [1, ceil(N / 128)]; returns 1 for N < 1. Following the kaispace blog
 * (section 4.2), the split count is a grid-dimension choice; here a fixed
 * rule picks it instead of a search. */
int mga_gqa_choose_splits(int B, int M, int N, int D);

/* The split count actually launched for a requested `splits` (0 = policy);
 * the grid dimension and for-loop range of the kaispace blog, section 4.2:
 * the chunk is ceil(ceil(N/128) / splits) key blocks and the count is
 * ceil(ceil(N/128) / chunk), so that no split is empty. Returns -1 for
 * arguments mga_gqa_check_args would reject with INVALID_VALUE or CONFIG. */
int mga_gqa_effective_splits(int B, int M, int N, int D, int splits);

/* Bytes of workspace mga_gqa_forward needs. It plays the role of the runtime
 * buffer `buf` that the generated host entry receives (Mirage documentation,
 * "Generated CUDA Code Example") and whose size the CUDA transpiler reports
 * (kaispace blog, section 5.2). With an effective split count
 * s > 1, the normalised partials o[s][B][M][D] in fp16 (s*B*M*D*2 bytes,
 * rounded up to 256) followed by the denominators L[s][B][M] in fp32
 * (s*B*M*4 bytes), rounded up to 256; then, when N % 8 != 0, the copy of K
 * with rows of ceil8(N) keys (B*D*ceil8(N)*2 bytes, rounded up to 256). 0
 * when neither applies. Its contents need no initialisation. Returns 0 for
 * invalid shapes. Enough for mga_gqa_forward_strided too (which never copies
 * K). */
size_t mga_gqa_workspace_bytes(int B, int M, int N, int D, int splits);

/* The launch geometry the library picks (host only): query rows per
 * workgroup and the effective split count, i.e. the block-grid shape and the
 * for-loop range that the kaispace blog (section 4.2) lists as search
 * parameters, chosen here by a fixed rule. With C the compute units of the current
 * device (256 on MI355X; see "Chip size" above): D = 64: 256 or 128 rows
 * when that tile alone gives at least C workgroups (one per compute unit),
 * else 256 rows when two splits do, else 64 rows, or 32 rows when even the
 * most splits leave 64-row tiles short of C workgroups (and always for
 * M <= 32); D = 128: 32 rows. Splits then bring the grid to C workgroups (2C
 * for 32-row tiles at D = 64, two of which share a compute unit), each keeping
 * at least 4 blocks of 128 keys. Either output pointer
 * may be NULL. Returns MGA_OK, INVALID_VALUE or CONFIG for the shape; the
 * memory layout is not part of the plan. */
int mga_gqa_plan(int B, int M, int N, int D, int splits, int *tile_rows, int *eff_splits);

/* Host-only validation of a forward call, the counterpart of compile()'s
 * check that run-time tensors match the graph's shapes and strides (kaispace
 * blog, section 2); launches nothing (its one runtime query is the chip size,
 * see "Chip size" above), so it is usable without a GPU. Returns the status
 * mga_gqa_forward would return before launching. `ws` may be NULL when the
 * effective split count is 1. B == 0 or M == 0 is valid (a no-op). */
int mga_gqa_check_args(const void *q, const void *k, const void *v, const void *o,
                       int B, int M, int N, int D, int splits, const void *ws, size_t ws_bytes);

/* The whole path (the graph of the Mirage documentation page "Mirage: Define
 * GQA Computation Graph", evaluated as the for-loop-accumulate plus combine
 * form of the kaispace blog, sections 2.1 and 4.2-4.3): partial kernel, then
 * (when the effective split count is above 1) the combine kernel, both on
 * `stream`. splits = 0 lets the policy
 * choose. ws/ws_bytes: caller-owned device workspace of at least
 * mga_gqa_workspace_bytes(B, M, N, D, splits) bytes, 16-byte aligned. Calls
 * that share a workspace must not overlap in time. */
int mga_gqa_forward(const void *q, const void *k, const void *v, void *o,
                    int B, int M, int N, int D, int splits, void *ws, size_t ws_bytes,
                    void *stream);

/* mga_gqa_forward on strided views: graph inputs declared with other strides
 * (kaispace blog, section 2: new_input accepts explicit strides), e.g. K as the
 * transpose of a [keys][head dim] cache, or K and V interleaved in one cache. `strides` points to nine element strides
 * (not bytes), in this order:
 *     q_b, q_i          Q[b][i][d] at q + b*q_b + i*q_i + d
 *     k_b, k_d, k_n     K[b][d][n] at k + b*k_b + d*k_d + n*k_n
 *     v_b, v_n          V[b][n][d] at v + b*v_b + n*v_n + d
 *     o_b, o_i          O[b][i][d] at o + b*o_b + i*o_i + d
 * NULL means contiguous (the call is then mga_gqa_forward). Accepted
 * layouts (else MGA_ERR_LAYOUT):
 *   - K head-dim-major (k_n == 1, k_d >= N) or key-major (k_d == 1,
 *     k_n >= D);
 *   - every stride other than those unit strides a non-negative multiple of
 *     8 elements, row strides q_i, v_n, o_i >= D, and O's batches disjoint
 *     (o_b >= (M - 1) o_i + D when B > 1); Q, K and V may overlap or be
 *     shared across batches (stride 0).
 * N may then be any value from 1 to 2^30 / D - 1 (keys past N in a padded
 * head-dim-major row are never used). Strides above 2^30 (rows) or 2^48
 * (batches), or a batch's K or V, or a workgroup's Q rows, spanning 2^31
 * bytes or more, give MGA_ERR_CONFIG. Same workspace as mga_gqa_forward. */
int mga_gqa_forward_strided(const void *q, const void *k, const void *v, void *o,
                            int B, int M, int N, int D, const int64_t *strides, int splits,
                            void *ws, size_t ws_bytes, void *stream);

/* Host-only validation of a mga_gqa_forward_strided call (launches
 * nothing); the shape and stride check of compile() (kaispace blog,
 * section 2). */
int mga_gqa_check_args_strided(const void *q, const void *k, const void *v, const void *o,
                               int B, int M, int N, int D, const int64_t *strides, int splits,
                               const void *ws, size_t ws_bytes);

/* Only the split-KV partial kernel (the for-loop over keys with
 * accumulation, kaispace blog sections 2.1 and 4.2: forloop_dim / fmap over
 * the key dimension; preceded by the K copy when N % 8 != 0). With one effective split it writes O directly
 * (normalised, fp16); otherwise it writes the normalised partials and
 * denominators into `ws` and leaves `o` untouched. Same arguments and checks
 * as mga_gqa_forward. */
int mga_gqa_partial(const void *q, const void *k, const void *v, void *o,
                    int B, int M, int N, int D, int splits, void *ws, size_t ws_bytes,
                    void *stream);

/* Only the combine kernel (the second block graph that sums the grid blocks'
 * partial results, kaispace blog sections 2.1 and 4.5, partial_sum /
 * combine):
 *     O[b,i,:] = fp16(sum_s L[s,b,i] o[s,b,i,:] / sum_s L[s,b,i])
 * with the sums taken in fp32 in a fixed order (split order; from 32 splits,
 * four contiguous quarters in split order, then the quarters in order). `ws` holds the partials a preceding
 * mga_gqa_partial call wrote for the same (B, M, N, splits); q, k and v are
 * not read. A no-op returning MGA_OK when the effective split count is 1. */
int mga_gqa_combine(void *o, int B, int M, int N, int D, int splits,
                    const void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and arguments as mga_gqa_forward_strided (strides NULL =
 * contiguous; splits 0 = policy), with no workspace argument. The workspace
 * the plan needs (mga_gqa_workspace_bytes) comes from one device scratch
 * array of MGA_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU that the library owns:
 * it is part of the library's code object, so it exists from the library's
 * first use on that GPU until the process ends, and this call allocates and
 * frees nothing (its address is looked up once per device, on the first
 * call with that device current). A plan that needs more than the scratch
 * returns MGA_ERR_SCRATCH and launches nothing. Every call on one GPU shares
 * that GPU's scratch, which keeps the last call's contents (nothing in it
 * needs clearing): calls that overlap in time on one GPU race and give
 * undefined results, so the caller serialises them (e.g. one stream). */
#define MGA_NOALLOC_SCRATCH_BYTES (16u << 20)
int mga_gqa_forward_noalloc(const void *q, const void *k, const void *v, void *o,
                            int B, int M, int N, int D, const int64_t *strides, int splits,
                            void *stream);

/* ---- QK-normalised variant ---------------------------------------------
 * Attention with QK normalisation (Mirage documentation tutorial "Implement
 * QK Normalization and Optimize Attention Kernel in Python", the
 * attention-with-kv-norm page): Q = rms_norm(Q), K = rms_norm(K), then the
 * same graph. The pages leave rms_norm's axis, eps and weight open; here every
 * query row and every key vector (a column of head-dim-major K) is divided by
 * the root mean square of its D entries, eps added inside the root, no weight:
 *     q-hat = q / sqrt(mean_d q_d^2 + eps),  k-hat likewise per key,
 *     O = softmax over keys of (q-hat . k-hat) applied to V.
 * After normalisation |q-hat . k-hat| reaches D, far past fp16 for exp, so
 * this path keeps a per-row reference maximum and rescales (exact: E / S is
 * unchanged by a common factor); partials carry log2 of their weight mass.
 * Numerics: q-hat is rounded to fp16 (with log2(e) folded in) as the graph's
 * fp16 tensor is; key norms scale the fp32 scores. eps must be finite and
 * >= 0 (else MGA_ERR_INVALID_VALUE); eps = 0 with an all-zero vector gives
 * NaN, as the definition does. Same layouts, strides (NULL = contiguous),
 * status codes and ownership as mga_gqa_forward_strided; the kernel shape is
 * 32 rows (M <= 32 or D = 128) or 64 rows per workgroup, so the split policy
 * and workspace size may differ from the plain path's. */
int mga_gqa_qknorm_forward(const void *q, const void *k, const void *v, void *o,
                           int B, int M, int N, int D, float eps, const int64_t *strides,
                           int splits, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes mga_gqa_qknorm_forward needs (same form as
 * mga_gqa_workspace_bytes, for this path's split count; the runtime buffer of
 * the kaispace blog, section 5.2); 0 for invalid shapes or one split. */
size_t mga_gqa_qknorm_workspace_bytes(int B, int M, int N, int D, int splits);

/* Tile rows and effective split count of the QK-normalised path (as
 * mga_gqa_plan; kaispace blog, section 4.2). */
int mga_gqa_qknorm_plan(int B, int M, int N, int D, int splits, int *tile_rows, int *eff_splits);

/* Host-only validation of a mga_gqa_qknorm_forward call (launches nothing;
 * the compile()-time shape and stride check, kaispace blog section 2). */
int mga_gqa_qknorm_check_args(const void *q, const void *k, const void *v, const void *o,
                              int B, int M, int N, int D, float eps, const int64_t *strides,
                              int splits, const void *ws, size_t ws_bytes);

#ifdef __cplusplus
}
#endif

#endif /* MGA_GQA_H */
