/*
 * qmm.h -- quantized matrix products with inline dequantization, for AMD
 * Instinct MI355X (gfx950).  Plain C ABI: no HIP, torch or C++ types.
 *
 * The operation (from the pages):
 *   Weights are stored with affine quantization at 2 to 8 bits per weight
 *   ("Apple Silicon 로컬 LLM 추론의 새 기준 BaseRT" (thakicloud.com), section
 *   "BaseRT는 무엇인가").  Decode multiplies one activation row by the
 *   weights with a dedicated GEMV (M = 1) and prefill several rows with a
 *   GEMM (M > 1); dequantization happens inside the compute loop, so full
 *   precision weights never go to memory and memory traffic scales with the
 *   compressed size ("BaseRT claims fastest Apple Silicon inference"
 *   (thetesserapress.com), section "What BaseRT does differently"; "BaseRT:
 *   Best-in-Class LLM Inference on Apple Silicon via Native Metal"
 *   (gist.science summary), section "Metodologia", per-format GEMV/GEMM
 *   variants with dequantization in the inner loop).
 *
 * Format (the pages fix none of these details; this is the library's format):
 *   W is N x K (output rows x reduction).  Codes are unsigned b-bit integers,
 *   b in {2, 3, 4, 5, 6, 8}.  Row n is a little-endian bitstream of K*b bits held
 *   in K*b/32 uint32 words: code k occupies stream bits [k*b, k*b + b), and
 *   stream bit i is bit (i mod 32) of word floor(i / 32) of the row.  Rows are
 *   contiguous (row n starts at word n*K*b/32).
 *   Each run of `group_size` consecutive k of a row shares one fp16 scale s
 *   and one fp16 min m, stored as two arrays [N][K/group_size] row-major.
 *   The weight is w[n][k] = s[n][k/group_size] * q[n][k] + m[n][k/group_size].
 *   Activations x are fp16 [M][K] row-major; outputs y are fp32 [M][N]
 *   row-major:  y[i][n] = sum_k w[n][k] * x[i][k].
 *   bits = 16 is the unquantized format ("FP16"/"Q16" in the per-format
 *   kernel lists of the pages above): w_packed holds the fp16 weights
 *   themselves, K/2 words per row, word j holding k = 2j in its low 16 bits
 *   and k = 2j + 1 in its high 16 bits.  Scales and mins are not read and may
 *   be NULL; group_size is still checked as above.  qmm_unpack rejects it
 *   (QMM_ERR_UNSUPPORTED), and a batched launch covers K <= 4096 at 16 bits.
 *
 * Requirements checked on the host before anything is launched:
 *   bits in {2, 3, 4, 5, 6, 8, 16} (7 is QMM_ERR_UNSUPPORTED); group_size a
 *   positive multiple of 32;
 *   k >= 32 and k a multiple of group_size; n >= 0, m >= 0 (0 is a no-op);
 *   weight, activation and output pointers 16-byte aligned; scale and min
 *   pointers 2-byte aligned; non-NULL pointers wherever work is to be done.
 *   One packed matrix (one expert of a stack) and one activation block must
 *   each stay below 4 GiB, else QMM_ERR_UNSUPPORTED (the kernels address
 *   them with 32-bit offsets); so must one output block.
 *   A failed check returns a status, writes nothing and launches nothing;
 *   qmm_last_error() then holds a one-line explanation (thread-local).
 *
 * Memory and streams:
 *   Every pointer argument except those marked "host" is a device pointer,
 *   owned by the caller.  The library allocates no device memory, frees none
 *   and keeps no per-call state.  Calls are asynchronous on `stream`
 *   (a hipStream_t passed as void*; NULL means the null stream); a kernel
 *   fault shows up at the caller's next synchronization.  Results are
 *   deterministic -- every output element is summed in a fixed order that
 *   depends only on the shape and the launch plan -- except for
 *   qmm_moe_combine, whose float atomic adds into a token's row happen in
 *   no fixed order.  The one exception to "allocates nothing" is
 *   qmm_gemm_noalloc's fixed scratch array (see there).
 *   The launch plan (kernel variant, tiles, splits, grids) depends on the
 *   shape, the bit width and the device's compute-unit count, and on the
 *   overrides of qmm_set_override, which the library reads from the
 *   environment once, when it is loaded; no call reads the environment.
 *   QMM_ERR_DEVICE is returned when the HIP runtime reports an error at
 *   launch time, or when no GPU is present.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMM_ABI_VERSION 3

#if defined(__GNUC__) || defined(__clang__)
#define QMM_API __attribute__((visibility("default")))
#else
#define QMM_API
#endif

typedef enum qmm_status {
    QMM_OK = 0,
    QMM_ERR_INVALID_ARGUMENT = 1, /* shape, size or NULL pointer problem      */
    QMM_ERR_UNSUPPORTED = 2,      /* valid request the library does not cover */
    QMM_ERR_MISALIGNED = 3,       /* pointer alignment below the requirement  */
    QMM_ERR_DEVICE = 4            /* HIP runtime error at launch / no device  */
} qmm_status;

/* Decode GEMV (M = 1): y[n] = sum_k (s*q + m)[n][k] * x[k].
 * Pages: "BaseRT claims fastest Apple Silicon inference", section "What
 * BaseRT does differently" (dedicated GEMV kernels for decode where M = 1,
 * dequantization inline in the compute loop).
 *   w_packed  uint32 [n][k*bits/32]      scales, mins  fp16 [n][k/group_size]
 *   x         fp16   [k]                 y             fp32 [n] (written)     */
QMM_API qmm_status qmm_gemv(const void *w_packed, const void *scales, const void *mins,
                    const void *x, float *y, int64_t n, int64_t k,
                    int bits, int group_size, void *stream);

/* Decode GEMV with the residual add fused into its epilogue:
 *   y[n] = residual[n] + sum_k (s*q + m)[n][k] * x[k].
 * Pages: "BaseRT claims fastest Apple Silicon inference", section "What
 * BaseRT does differently" (fusion removes a launch and a global-memory round
 * trip per fusion; residual buffers are part of the decode loop's state).
 *   residual fp32 [n], 4-byte aligned, non-NULL; it may be y itself (y +=
 *   W x: each row's residual is read before that row is written).  Other
 *   arguments as qmm_gemv.                                                  */
QMM_API qmm_status qmm_gemv_residual(const void *w_packed, const void *scales,
                                     const void *mins, const void *x, const float *residual,
                                     float *y, int64_t n, int64_t k, int bits, int group_size,
                                     void *stream);

/* Fused gate/up projection of a feed-forward block (decode, M = 1):
 *   h[n] = silu(g[n]) * u[n],  g = Wg x,  u = Wu x,  silu(v) = v / (1 + e^-v).
 * Pages: "BaseRT claims fastest Apple Silicon inference", section "What
 * BaseRT does differently" (kernel fusion removes a launch and a global
 * memory round trip per fusion); "BaseRT: Best-in-Class LLM Inference on
 * Apple Silicon via Native Metal", section "Metodologia" (operator sequences
 * of feed-forward blocks fused into one kernel).
 * Both matrices are n x k in the same format (bits, group_size) with their
 * own scale and min arrays; g and u stay in registers, only h is written.
 *   x fp16 [k]      h fp32 [n] (written)
 * k must fit one pass of the decode kernel (k <= 8192 codes for 64-multiple
 * groups, 4096 for 32-code groups and for fp16 weights), else
 * QMM_ERR_UNSUPPORTED.                                                      */
QMM_API qmm_status qmm_gemv_swiglu(const void *gate_w, const void *gate_scales,
                                   const void *gate_mins, const void *up_w,
                                   const void *up_scales, const void *up_mins,
                                   const void *x, float *h, int64_t n, int64_t k,
                                   int bits, int group_size, void *stream);

/* Prefill GEMM (M >= 1): y[i][n] = sum_k (s*q + m)[n][k] * x[i][k].
 * Pages: "BaseRT claims fastest Apple Silicon inference", section "What
 * BaseRT does differently" (GEMM kernels for prefill where M > 1); "BaseRT:
 * Best-in-Class LLM Inference on Apple Silicon via Native Metal", section
 * "Metodologia" (tiled prefill GEMM on the GPU's matrix units).
 * The weights are dequantized to fp16 tiles and multiplied on fp16 matrix
 * cores with fp32 accumulation.  Small m is routed to the bandwidth-bound
 * multi-row GEMV kernel.
 *   x  fp16 [m][k]      y  fp32 [m][n] (written)
 *   workspace: optional device scratch (may be NULL / 0 bytes), 16-byte
 *   aligned.  When the shape leaves the GPU under-filled, up to
 *   qmm_gemm_workspace_bytes() of it is used to split the K loop; with less,
 *   the split shrinks to what fits (no split with none).  Its first 4096
 *   bytes hold per-tile arrival counters: the workspace must be all zero before
 *   its first use (allocate it zeroed once), and every call leaves those
 *   counters zero again, so one workspace serves any sequence of calls on
 *   one stream.  Calls that overlap (other streams) need their own
 *   workspace.  The rest of its contents on return are unspecified.
 *   Two-way splits are summed inside the GEMM kernel: each work-group
 *   writes its partial sums with stores that go through every cache to
 *   memory (the system-coherent cache policy of gfx950 buffer stores),
 *   waits until they are acknowledged, then bumps its tile's counter with a
 *   relaxed device-scope atomic add; the work-group that arrives last reads
 *   the partial sums with loads that bypass the caches, writes y and resets
 *   the counter.  Correctness rests on those cache-policy bits and the
 *   store acknowledgement, not on release/acquire fences (a device-scope
 *   fence would write back and invalidate a whole L2 per wave).  Larger
 *   splits are summed by a second kernel on the same stream.               */
QMM_API qmm_status qmm_gemm(const void *w_packed, const void *scales, const void *mins,
                    const void *x, float *y, int64_t m, int64_t n, int64_t k,
                    int bits, int group_size, void *workspace,
                    size_t workspace_bytes, void *stream);

/* Prefill GEMM with fp16 output: y[i][n] as qmm_gemm, rounded once from the
 * fp32 sums to fp16 (nearest even; beyond the fp16 range +-inf).  Halves the
 * output bytes for long prefills ("BaseRT: Best-in-Class LLM Inference on
 * Apple Silicon via Native Metal", section "Resultados": prefill measured at
 * 2048 tokens).  Every m runs on the matrix-core kernel; workspace as for
 * qmm_gemm (split partial sums stay fp32; qmm_gemm_workspace_bytes gives the
 * preferred size for m > 2, none is needed below that).
 *   y  fp16 [m][n] (written), 16-byte aligned.                             */
QMM_API qmm_status qmm_gemm_f16out(const void *w_packed, const void *scales,
                                   const void *mins, const void *x, void *y, int64_t m,
                                   int64_t n, int64_t k, int bits, int group_size,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Prefill GEMM that allocates nothing, for callers that cannot call
 * hipMalloc or take a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.
 * Same arguments and result as qmm_gemm without the workspace: it runs the
 * plan qmm_gemm takes with its preferred workspace (qmm_gemm_workspace_bytes),
 * so y is bit-identical to that call's.  The K-split partial sums and
 * arrival counters live in a static device array of
 * QMM_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends; a shape that would need more (qmm_gemm_workspace_bytes
 * above that) returns QMM_ERR_UNSUPPORTED and launches nothing.  Each call
 * resets the counters it uses with a small kernel before the GEMM (no
 * memset, no allocation).  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other host threads) race
 * and give wrong results; calls ordered on one stream are safe.           */
#define QMM_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)

QMM_API qmm_status qmm_gemm_noalloc(const void *w_packed, const void *scales, const void *mins,
                                    const void *x, float *y, int64_t m, int64_t n, int64_t k,
                                    int bits, int group_size, void *stream);

/* Grouped prefill GEMM: up to 4 weight matrices that share the activations
 * x [m][k] (the q, k and v projections of a layer, or gate and up), one
 * launch: y_i[r][j] = sum_k (s*q + m)_i[j][k] * x[r][k] for every member i.
 * Pages: "BaseRT claims fastest Apple Silicon inference", section "What
 * BaseRT does differently" (operations other runtimes dispatch separately
 * run as one fused dispatch; GEMM kernels for prefill).
 *   members (host array of count, 1..4): each member's packed weights,
 *     scales and mins in the qmm_gemm layout with its own n (n == 0: the
 *     member is skipped), and its output y fp32 [m][n], 16-byte aligned.
 *   x fp16 [m][k], 16-byte aligned; bits and group_size shared.
 *   workspace: as qmm_gemm (zero before its first use, counters left zero);
 *     qmm_gemm_grouped_workspace_bytes gives the preferred size (it reads
 *     the members' n only; sized for the current device, or for 256
 *     compute units where no device can be queried).
 * The library chooses between one launch and one launch per member (as
 * qmm_gemm would, same stream, same workspace) from the shapes: one launch
 * where the members underfill the GPU on their own, or where their tiles
 * together fill it without a K split; separate launches where each
 * member's own tile grid fills it.  Either way each y_i is member i's
 * product to qmm_gemm's accuracy.  A grouped launch sums any K split
 * inside the kernel, as described for two-way splits under qmm_gemm.      */
typedef struct {
    const void *w_packed;
    const void *scales;
    const void *mins;
    float *y;
    int64_t n;
} qmm_gemm_member;

QMM_API qmm_status qmm_gemm_grouped(const qmm_gemm_member *members, int count, const void *x,
                                    int64_t m, int64_t k, int bits, int group_size,
                                    void *workspace, size_t workspace_bytes, void *stream);
QMM_API size_t qmm_gemm_grouped_workspace_bytes(const qmm_gemm_member *members, int count,
                                                int64_t m, int64_t k, int bits, int group_size);

/* Many independent decode GEMVs in one launch.
 * Pages: "BaseRT claims fastest Apple Silicon inference", section "What
 * BaseRT does differently" (operations other runtimes dispatch separately
 * are combined, saving launches); "BaseRT: Best-in-Class LLM Inference on
 * Apple Silicon via Native Metal", section "Metodologia" (low-overhead
 * dispatch without per-operation scheduling).
 * Every descriptor is one qmm_gemv (same bits and group_size for all; each
 * k at most 8192 codes for 64-multiple groups, 4096 otherwise and at 16
 * bits, else QMM_ERR_UNSUPPORTED; the whole batch below 2^31 row batches,
 * likewise).  Launch start-up reads a 256-entry index of the work list from
 * the kernel arguments, so finding a wave's first descriptor costs one
 * dependent load of the device copy whatever the count.  first_item is owned by
 * the library: qmm_gemv_batch_prepare fills it in a host array, the caller
 * copies the array to device memory (once; it can be reused for every
 * later call with the same shapes and pointers) and passes both copies to
 * qmm_gemv_batched, which checks the host copy and launches one kernel that
 * reads the device copy.  The two copies must hold the same bytes.  Outputs
 * of different descriptors must not overlap.                                */
typedef struct qmm_gemv_desc {
    const void *w_packed;   /* uint32 [n][k*bits/32]                          */
    const void *scales;     /* fp16 [n][k/group_size]                         */
    const void *mins;       /* fp16 [n][k/group_size]                         */
    const void *x;          /* fp16 [k]                                       */
    float *y;               /* fp32 [n] (written)                             */
    int64_t n, k;
    int64_t first_item;     /* library-owned, see qmm_gemv_batch_prepare      */
} qmm_gemv_desc;

QMM_API qmm_status qmm_gemv_batch_prepare(qmm_gemv_desc *descs /* host */, int64_t count,
                                          int bits, int group_size);
QMM_API qmm_status qmm_gemv_batched(const qmm_gemv_desc *descs_device,
                                    const qmm_gemv_desc *descs_host, int64_t count,
                                    int bits, int group_size, void *stream);

/* Bytes of workspace that let qmm_gemm use its preferred K split for this
 * shape on the current device (0 when it would not split; sized for 256
 * compute units where no device can be queried).  Host only.              */
QMM_API size_t qmm_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int bits,
                                int group_size);

/* Mixture-of-experts projection over rows grouped by expert.
 * Pages: "BaseRT claims fastest Apple Silicon inference", section "Where the
 * wins land, and where they don't" (MoE decode and prefill; routing handled
 * without branching in the hot path); "BaseRT: Best-in-Class LLM Inference on
 * Apple Silicon via Native Metal", section "Resultados" (MoE prefill).
 *   w_packed  uint32 [n_experts][n][k*bits/32]  (experts stacked)
 *   scales, mins fp16 [n_experts][n][k/group_size]
 *   expert_offsets int32 [n_experts + 1] (device): rows of expert e are
 *     p in [expert_offsets[e], expert_offsets[e+1]); non-decreasing, from 0
 *     to p_rows.
 *   x fp16 [x_rows_count][k]; x_rows int32 [p_rows] (device) or NULL:
 *     row p of the product reads activation row x_rows[p] (row p if NULL).
 *   y fp32 [p_rows][n] (written): y[p][j] = sum_k w_e[j][k] * x[row(p)][k].
 * Rows whose activation index is outside [0, x_rows_count) are written as
 * NaN (nothing is read out of bounds); output rows that no expert range
 * covers are left untouched.  Offsets are clamped to [0, p_rows].  Routing
 * weights are not applied.                                                 */
QMM_API qmm_status qmm_moe_gemm(const void *w_packed, const void *scales, const void *mins,
                        const void *x, const int32_t *x_rows, int64_t x_rows_count,
                        const int32_t *expert_offsets, float *y, int64_t p_rows,
                        int64_t n_experts, int64_t n, int64_t k, int bits,
                        int group_size, void *stream);

/* Fused gate/up projection of the selected experts:
 *   h[p][j] = silu(g[p][j]) * u[p][j], g and u as qmm_moe_gemm over the
 *   gate stack and the up stack, silu(v) = v / (1 + e^-v).
 * Pages: as qmm_gemv_swiglu (fusion of feed-forward operator sequences) and
 * as qmm_moe_gemm (expert rows).  Both stacks [n_experts][n][...] in one
 * format; the remaining arguments and the NaN rule are those of
 * qmm_moe_gemm.  k must fit one pass (as qmm_gemv_swiglu), else
 * QMM_ERR_UNSUPPORTED.                                                      */
QMM_API qmm_status qmm_moe_swiglu(const void *gate_w, const void *gate_scales,
                                  const void *gate_mins, const void *up_w,
                                  const void *up_scales, const void *up_mins, const void *x,
                                  const int32_t *x_rows, int64_t x_rows_count,
                                  const int32_t *expert_offsets, float *h, int64_t p_rows,
                                  int64_t n_experts, int64_t n, int64_t k, int bits,
                                  int group_size, void *stream);

/* Expert projection with the routing-weighted combine fused into its store:
 *   y[pair_token[p]][j] += pair_weight[p] * sum_k w_e[j][k] * x[row(p)][k]
 * for every row p of expert e, so each token's row of y receives the
 * weighted sum of its selected experts' outputs (the MoE down projection and
 * combine in one launch; y may hold the residual stream beforehand).
 * Pages: as qmm_moe_gemm (expert rows) and as qmm_gemv_swiglu (fusion of
 * operator sequences saves a launch and a round trip through memory).
 *   pair_token int32 [p_rows], pair_weight fp32 [p_rows] (device, 4-byte
 *     aligned): token and routing weight of row p.
 *   y fp32 [n_tokens][n], 16-byte aligned, read and written (accumulated).
 * Other arguments as qmm_moe_gemm.  The adds into one element of y happen in
 * no fixed order (float atomics), so results may differ in the last bits
 * from run to run.  Rows with an activation index out of range add NaN to
 * their token's row; rows whose token is outside [0, n_tokens) add nothing.
 * n_tokens == 0 or p_rows == 0 is a no-op.                                  */
QMM_API qmm_status qmm_moe_combine(const void *w_packed, const void *scales, const void *mins,
                                   const void *x, const int32_t *x_rows, int64_t x_rows_count,
                                   const int32_t *expert_offsets, const int32_t *pair_token,
                                   const float *pair_weight, float *y, int64_t n_tokens,
                                   int64_t p_rows, int64_t n_experts, int64_t n, int64_t k,
                                   int bits, int group_size, void *stream);

/* Codes as bytes: codes[n][k] = q[n][k] (uint8).  Bit-exact view of the
 * packed format, used to check the GPU's bit extraction.                   */
QMM_API qmm_status qmm_unpack(const void *w_packed, uint8_t *codes, int64_t n, int64_t k,
                      int bits, void *stream);

/* Launch plan the library would use (host only, no device call): which
 * kernel variant, grid and block.  `op` is 0 for qmm_gemv, 1 for qmm_gemm,
 * 2 for qmm_moe_gemm (m = rows per expert bound), 3 for qmm_gemv_batched
 * (n = total rows of the batch, k = its largest k).  cu_count <= 0 means
 * "query the current device" (then this does call the runtime).            */
typedef struct qmm_plan {
    int32_t variant;       /* library-internal variant id                   */
    int32_t lanes_per_row; /* GEMV: lanes cooperating on one output row     */
    int32_t units_per_lane;/* GEMV: 64- or 32-code units per lane per pass  */
    int32_t rows_per_iter; /* GEMV: rows per lane slot per loop iteration   */
    int32_t unit_codes;    /* GEMV: codes per unit (64 or 32)               */
    int32_t split_k;       /* GEMM: K split (1 = none)                      */
    int32_t tile_m, tile_n;/* GEMM: block tile                              */
    int64_t grid;          /* work-groups launched                          */
    int32_t block;         /* threads per work-group                        */
    int32_t reserved[5];   /* GEMV: [0] multi-pass rows, [1] row sums staged
                              in LDS, [2] activation units built after the
                              first weight loads; the rest zero              */
} qmm_plan;

QMM_API qmm_status qmm_get_plan(int op, int64_t m, int64_t n, int64_t k, int bits,
                        int group_size, int cu_count, size_t workspace_bytes,
                        qmm_plan *plan /* host */);

/* Launch-plan override for measurement sweeps and for tests that force a
 * kernel variant (host only, process-wide, not meant for production: a
 * forced variant may be slower, and a value the chosen kernel cannot take
 * is ignored).  name is one of QMM_UNIT, QMM_GEMV_LPR, QMM_GEMV_XC,
 * QMM_GEMV_U, QMM_GEMV_WAVES_PER_CU, QMM_BATCH_U, QMM_ROWS_MR,
 * QMM_ROWS_WAVES_PER_CU, QMM_GEMM_TILE_M, QMM_GEMM_TILE_N, QMM_GEMM_SPLIT,
 * QMM_GEMM_WIDE_SCALES, QMM_GEMM_ORDER, QMM_GEMM_GROUPED, QMM_GEMM_KERNEL
 * (1: the prefill GEMM that dequantizes into LDS, 2: the one that
 * dequantizes into registers), QMM_GEMV_STAGED (1/0: single GEMVs with
 * 64-lane rows do / do not stage their row sums in LDS), QMM_GEMV_LATE
 * (1/0: single Q4 GEMVs of one unit per lane on at most 32 lanes do / do
 * not build their activation units after the first weight loads); value < 0 removes
 * the override.  The same names are read from the environment once, when
 * the library is loaded.  Unknown name: QMM_ERR_INVALID_ARGUMENT.          */
QMM_API qmm_status qmm_set_override(const char *name, int value);

QMM_API const char *qmm_status_string(qmm_status s);
QMM_API const char *qmm_last_error(void);   /* thread-local; "" when none */
QMM_API int qmm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
