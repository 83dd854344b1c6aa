/*
 * gemm355.h -- C ABI of libgemm355, a GEMM library for the AMD Instinct
 * MI355X (gfx950).
 *
 * The operation (phobos docs, page "gemm, f32", opening paragraph and section
 * "The epilogue"):
 *
 *     C = alpha * A @ B + beta * C
 *
 * with A an M x K, B a K x N and C an M x N matrix of f32, alpha and beta f32
 * scalars.  The f16r mode (phobos docs, page "gemm on tensor cores", section
 * "What changes") rounds every element of A and B to IEEE binary16 (round to
 * nearest, ties to even, subnormals kept) before multiplying and accumulates
 * the products in f32; C, alpha and beta stay f32.
 *
 * Layout and ownership (both modes):
 *   - all matrices are row-major: A[i*lda + k], B[k*ldb + j], C[i*ldc + j];
 *   - A, B and C are device pointers owned by the caller; A and B are only
 *     read; C is read (unless beta == 0) and written in place; C must not
 *     overlap A or B;
 *   - alpha and beta are host values passed by value.
 *
 * Execution:
 *   - the work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns without waiting for it;
 *   - the f16r mode writes the rounded operands, and configurations that
 *     split K over workgroups (both modes) write partial tiles and per-tile
 *     arrival counters, into device scratch that the library keeps in a pool
 *     per device (at most 8 buffers kept, each as large as the largest call it
 *     served).  A call holds one pool buffer from its first launch until its
 *     last launch is enqueued, so calls from several host threads never share
 *     one in between.  A buffer goes to a later call on the same stream at
 *     once (stream order), to a call on another stream only once the work of
 *     its last call has completed.  Buffers are allocated and freed
 *     stream-ordered (hipMallocAsync / hipFreeAsync on the call's stream): no
 *     call waits on the host.  Each call works out how much scratch it needs
 *     before it launches anything, so a failed allocation (GEMM355_ERR_ALLOC)
 *     leaves C untouched;
 *   - under stream capture a call allocates nothing: it uses a pool buffer of
 *     its stream that is already large enough (run the call once on that
 *     stream first), else it returns GEMM355_ERR_CAPTURE; that buffer then
 *     belongs to the graph and is never reused or freed (gemm355_gemm_noalloc
 *     captures without this cost);
 *   - every call is thread-safe.
 *
 * Special cases, decided on the host before any launch:
 *   - M == 0 or N == 0: nothing to do, returns 0;
 *   - K == 0 or alpha == 0: C = beta * C, A and B are not read;
 *   - beta == 0: C is only written, never read (NaN in C does not survive).
 *
 * Return value:
 *   0              success (the work is enqueued);
 *   -p (p = 1..11)  argument p is invalid (1 M, 2 N, 3 K, 5 A, 6 lda, 7 B,
 *                  8 ldb, 10 C, 11 ldc), as in BLAS's xerbla convention;
 *                  nothing is launched and C is untouched;
 *   GEMM355_ERR_*  (below -100) a library-level failure;
 *   > 0            a hipError_t reported by the HIP runtime at launch.  Faults
 *                  inside a kernel surface at the caller's next synchronisation.
 */
#ifndef GEMM355_H
#define GEMM355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GEMM355_MODE_F32 0  /* plain f32 operands, f32 accumulation */
#define GEMM355_MODE_F16R 1 /* operands rounded to binary16 (RNE), f32 accumulation */

#define GEMM355_OK 0
#define GEMM355_ERR_CONFIG (-101)   /* tile configuration unknown or not compiled */
#define GEMM355_ERR_ALLOC (-102)    /* workspace or scratch allocation failed */
#define GEMM355_ERR_MODE (-103)     /* mode is neither F32 nor F16R */
#define GEMM355_ERR_BUFFER (-104)   /* output buffer too small */
#define GEMM355_ERR_INTERNAL (-105) /* no kernel instance fits (library bug) */
#define GEMM355_ERR_CAPTURE (-106)  /* scratch would have to be allocated during stream capture */
#define GEMM355_ERR_SCRATCH (-107)  /* larger than the fixed scratch of gemm355_gemm_noalloc */

/*
 * C = alpha*A@B + beta*C in f32.  Arguments:
 *   M, N, K   matrix sizes, each >= 0;
 *   A         device pointer to M x K f32, row stride lda >= max(1, K);
 *   B         device pointer to K x N f32, row stride ldb >= max(1, N);
 *   C         device pointer to M x N f32, row stride ldc >= max(1, N);
 *   stream    hipStream_t to enqueue on (NULL = default stream).
 * A and B may be NULL only when M*K (resp. K*N) is 0 or alpha == 0; C may be
 * NULL only when M*N is 0.
 */
int gemm_f32(int64_t M, int64_t N, int64_t K, float alpha,
             const float* A, int64_t lda, const float* B, int64_t ldb,
             float beta, float* C, int64_t ldc, void* stream);

/*
 * The same operation with A and B rounded to binary16 (round to nearest even)
 * and the products accumulated in f32 (phobos docs, "gemm on tensor cores",
 * section "What changes").  Arguments and return values as gemm_f32.
 */
int gemm_f16r_f32acc(int64_t M, int64_t N, int64_t K, float alpha,
                     const float* A, int64_t lda, const float* B, int64_t ldb,
                     float beta, float* C, int64_t ldc, void* stream);

/*
 * Operand layouts (the Matrix Multiplication lab, "Part 5", the layout sweep;
 * the transa/transb arguments of the BLAS GEMM interface the lab calls):
 *
 *     C = alpha * op(A) @ op(B) + beta * C
 *
 * with op(A) M x K and op(B) K x N:
 *   transa = 0: A is stored M x K, A[i*lda + k], lda >= max(1, K);
 *   transa = 1: A is stored K x M, op(A)[i][k] = A[k*lda + i], lda >= max(1, M);
 *   transb = 0: B is stored K x N, B[k*ldb + j], ldb >= max(1, N);
 *   transb = 1: B is stored N x K, op(B)[k][j] = B[j*ldb + k], ldb >= max(1, K).
 * Everything else (ownership, stream, special cases, rounding of the f16r
 * mode, which applies to the elements whatever their layout) is as for
 * gemm_f32 / gemm_f16r_f32acc, which are the transa = transb = 0 case.
 * Return codes follow BLAS sgemm's argument numbers: -1 transa, -2 transb
 * (not 0 or 1), -3 M, -4 N, -5 K, -7 A, -8 lda, -9 B, -10 ldb, -12 C,
 * -13 ldc; library errors and hipError_t values as gemm_f32.
 */
int gemm_f32_ex(int transa, int transb, int64_t M, int64_t N, int64_t K, float alpha,
                const float* A, int64_t lda, const float* B, int64_t ldb,
                float beta, float* C, int64_t ldc, void* stream);
int gemm_f16r_f32acc_ex(int transa, int transb, int64_t M, int64_t N, int64_t K, float alpha,
                        const float* A, int64_t lda, const float* B, int64_t ldb,
                        float beta, float* C, int64_t ldc, void* stream);

/*
 * The f16-output variant of the f16r mode (the Matrix Multiplication lab,
 * "Part 4 -- precision": FP16 operands and an FP16 result, half the bytes per
 * element of C): operands as in gemm_f16r_f32acc_ex (rounded to binary16,
 * products accumulated in f32); C16 is a device pointer to M x N IEEE
 * binary16 values (bit patterns, row stride ldc), read as binary16 when
 * beta != 0; alpha*acc + beta*C is evaluated in f32 and rounded once to
 * binary16, to nearest even (overflow to +-inf).  Arguments, special cases
 * and return codes as gemm_f16r_f32acc_ex (C16 is argument 12).  Tile choice,
 * pins and tuning are those of the f16r mode.
 */
int gemm_f16r_f16out(int transa, int transb, int64_t M, int64_t N, int64_t K, float alpha,
                     const float* A, int64_t lda, const float* B, int64_t ldb,
                     float beta, uint16_t* C16, int64_t ldc, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * variant of gemm_f32_ex (mode GEMM355_MODE_F32) and gemm_f16r_f32acc_ex
 * (mode GEMM355_MODE_F16R) that allocates no device memory.  Arguments,
 * special cases, results and return codes are those of the _ex entry point
 * of the mode (an invalid mode returns GEMM355_ERR_MODE).  Its scratch is one
 * fixed device array per GPU of 160 MiB (64 KiB of arrival counters, the rest
 * for packed operands and partial tiles), held from the first call on that
 * GPU until the process ends; the first call on a GPU looks up the array's
 * address there.  A call needing more returns GEMM355_ERR_SCRATCH with
 * nothing launched: the f16r mode packs 2 (M + N) K bytes of binary16
 * operands (M, N rounded up to 256, K to 64), and calls that split K over
 * workgroups keep up to 128 MiB of partial tiles (f16r 8192^3 or 3072^3, for
 * example, do not fit; 4096^3 does).  Every call on a GPU shares its
 * array, which keeps the last call's contents (the counters a call uses are
 * cleared by a kernel on its stream first): calls that overlap on one GPU,
 * from any stream or thread, race and must be ordered by the caller.
 */
int gemm355_gemm_noalloc(int mode, int transa, int transb, int64_t M, int64_t N, int64_t K,
                         float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                         float beta, float* C, int64_t ldc, void* stream);

/*
 * Per-shape tile autotuning (phobos docs, "gemm, f32", section "Tuning": time
 * every configuration briefly, skip those that fail, then re-time the fastest
 * few over interleaved rounds under the same clocks; a call under 0.2 ms is
 * timed as a batch of back-to-back calls, the time of a call in a stream of
 * calls).  Runs the candidates on
 * the caller's A and B and on a scratch C the library allocates and frees
 * (the caller's C is not touched), synchronises `stream`, and stores the
 * winner in the per-shape cache used by later calls with the same key
 * (mode, operand layout, M, N, K, alignment class of lda/ldb and pointers,
 * beta == 0).  `beta` only selects the key and the epilogue variant timed.
 * Returns 0, a negative argument code (numbered as the same argument of
 * gemm_f32), a library error, or a positive hipError_t.  gemm355_tune_ex takes
 * the operand layout as gemm_f32_ex and numbers its argument codes as there.
 */
int gemm355_tune(int mode, int64_t M, int64_t N, int64_t K,
                 const float* A, int64_t lda, const float* B, int64_t ldb,
                 float beta, int64_t ldc, void* stream);
int gemm355_tune_ex(int mode, int transa, int transb, int64_t M, int64_t N, int64_t K,
                    const float* A, int64_t lda, const float* B, int64_t ldb,
                    float beta, int64_t ldc, void* stream);

/*
 * The tile configuration a call with these arguments would use, written as
 * "BM=.. BN=.. BK=.. ST=.. WM=.. WN=.. GM=.." plus " source=pin|tuned|heuristic"
 * into buf (NUL-terminated, at most len bytes).  Host only; no GPU call.
 * gemm355_get_config_ex: the same for the operand layout (transa, transb).
 */
int gemm355_get_config(int mode, int64_t M, int64_t N, int64_t K,
                       int64_t lda, int64_t ldb, int64_t ldc, float beta,
                       char* buf, size_t len);
int gemm355_get_config_ex(int mode, int transa, int transb, int64_t M, int64_t N, int64_t K,
                          int64_t lda, int64_t ldb, int64_t ldc, float beta,
                          char* buf, size_t len);

/*
 * How a call with these arguments (operand pointers taken as 256-byte
 * aligned) would run, written into buf as "form=F block=MBxNBxKB" plus
 * " rows=4-byte" when a leading dimension keeps rows from being 16-byte
 * aligned.  F names the kernel path of the configuration gemm355_get_config_ex
 * reports: ring / ring-masked (the f32 ring of direct-to-LDS panel copies, in
 * every operand layout, on whole tiles or in its zero-filling form), tiles / tiles-masked (the
 * register-staged f32 kernel), packed / packed-masked (the f16r packing pass
 * and binary16 kernel, masked stores at ragged edges), split-k, rows,
 * columns (the few-rows configuration run on the transposed problem for a C
 * of at most 16 columns), round-on-load, panel-ring, and round-on-load-columns
 * / panel-ring-columns (the 16-row tile of the f32-panel ring run on the
 * transposed problem for a C of at most 16 columns, A stored M x K).  The block is the part
 * of C (MB x NB, over the first KB of K) that configuration runs itself; when
 * it is smaller than the call (the f32 ring, plain layout only), the right
 * strip, the bottom strip and the k tail run in the few-rows (or
 * few-columns), split-K or 64 x 64 configurations.  Host only; no GPU call.  Returns as
 * gemm355_get_config_ex.
 */
int gemm355_get_plan_ex(int mode, int transa, int transb, int64_t M, int64_t N, int64_t K,
                        int64_t lda, int64_t ldb, int64_t ldc, float beta, char* buf, size_t len);

/*
 * Pin one tile configuration for every later call of `mode`, skipping the
 * search (phobos docs, "gemm, f32", section "Tuning", the pinned run).
 * Grammar: space-separated KEY=VALUE with keys BM|TILE_M, BN|TILE_N,
 * BK|TILE_K, ST|STAGES, WM, WN, GM, KS|SPLITK; omitted keys take the first compiled
 * instance that matches the given ones, except KS, whose absence selects the
 * tiled configurations (KS=0).  KS=1: K split over workgroups, partial tiles
 * summed by a second pass; KS=2: one wavefront per few rows of C (a C of at
 * most 16 columns and more rows: per few columns, as the transposed problem
 * with C stored transposed); KS=3: K
 * split over workgroups and the slices added in order by the tile's last
 * workgroup, the operands staged as f32 panels from a ring of direct-to-LDS
 * copies (BK=32, both modes; in f16r rounded to binary16 as the fragments
 * are read, with no packing pass; its 16-row tile runs a C of at most 16
 * columns and more rows, with A stored M x K, as the transposed problem with
 * C stored transposed) or, in f16r only, rounded to binary16
 * through registers (BK=64).  A ring configuration (direct-to-LDS copies)
 * that a call's row alignment or shape rules out runs that call in a
 * register-staged kernel instead: the f32 one of the same tile, BM=64 BN=64
 * BK=64 KS=3 for the f16r panel ring, the split-K tiles (KS=1) for the f32
 * one.
 * NULL or "" clears the pin.  The environment
 * variables GEMM355_CONFIG_F32 / GEMM355_CONFIG_F16R set the initial pin.
 * Returns 0 or GEMM355_ERR_CONFIG (the pin is then unchanged).  Host only.
 */
int gemm355_set_config(int mode, const char* spec);

/*
 * Parse `spec` (grammar as gemm355_set_config) and write the canonical form of
 * the compiled instance it names into buf.  Returns 0 or GEMM355_ERR_CONFIG.
 * Host only.
 */
int gemm355_parse_config(int mode, const char* spec, char* buf, size_t len);

/*
 * Newline-separated canonical forms of every compiled tile configuration of
 * `mode`.  Returns the number of configurations, or a negative error.
 * Host only.
 */
int gemm355_list_configs(int mode, char* buf, size_t len);

/* Load (path != NULL) or save (path == NULL: to the same path) the per-shape
 * tuning cache as text.  Lines that do not parse or name unknown instances
 * are ignored.  Returns the number of entries read/written, or a negative
 * error.  Host only. */
int gemm355_cache_load(const char* path);
int gemm355_cache_save(const char* path);
/* Drop every tuned entry.  Host only. */
void gemm355_cache_clear(void);

/* Text for a status code returned by this library.  Never NULL. */
const char* gemm355_strerror(int status);

/* Library version string, e.g. "0.1.0". */
const char* gemm355_version(void);

/*
 * Measurement kernels for the roofs the GEMM is judged against (the
 * Matrix Multiplication lab, "Part 1 -- the two roofs, again": a kernel of
 * nothing but independent multiply-adds, and a streaming read).
 *
 * gemm355_roof_mfma: enqueue `blocks` workgroups of 256 threads, each wave
 * issuing `iters` rounds of independent matrix instructions of the mode in
 * one form (form 0: 8 instructions of 32x32 blocks per round, F32
 * v_mfma_f32_32x32x2_f32, F16R v_mfma_f32_32x32x16_f16; form 1: 16 of 16x16
 * blocks, v_mfma_f32_16x16x4_f32 / v_mfma_f32_16x16x32_f16, f32
 * accumulators) into `sink` (device, >= blocks*256 floats).  *flops_out
 * receives the flop count of the launch (2*m*n*k per instruction).
 *
 * gemm355_roof_fma: the same with vector f32 fused multiply-adds instead of
 * matrix instructions (8 independent chains per thread, one FMA per element:
 * no packed f32 instructions), the cross-check of the f32 matrix roof;
 * *flops_out receives 2 per FMA.
 *
 * gemm355_roof_hbm: enqueue a grid-stride 16-byte read of `bytes` bytes
 * (multiple of 16) from device pointer `buf`, with `blocks` workgroups of 256
 * threads; `sink` is a device float written only to keep the loads alive.
 *
 * gemm355_copy_f32: enqueue dst[i] = src[i] for n floats (a plain copy
 * kernel of known traffic, for calibrating hardware byte counters).
 */
int gemm355_roof_mfma(int mode, int form, int64_t iters, int blocks, float* sink,
                      double* flops_out, void* stream);
int gemm355_roof_fma(int64_t iters, int blocks, float* sink, double* flops_out, void* stream);
int gemm355_roof_hbm(const void* buf, int64_t bytes, int blocks, float* sink, void* stream);
int gemm355_copy_f32(const float* src, float* dst, int64_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM355_H */
