/*
 * libdpnorm: randomized per-sample gradient-norm estimation on MI355X (gfx950).
 *
 * The operations follow "Efficient DP-SGD for LLMs with Randomized Clipping"
 * (papernotes.org ICML 2026 note; gist.science/nl technical summary):
 *   - for a linear-like layer with hooked activations A_i (T x d) and output
 *     gradients G_i (T x p) of sample i, the squared per-sample gradient norm
 *     is ||A_i^T G_i||_F^2 = trace(G_i^T A_i A_i^T G_i) (note: 切入角度);
 *   - the Hutchinson estimate with a Gaussian projection P (p x k, entries of
 *     variance 1/k) is ||A_i^T (G_i P)||_F^2 (note: 关键设计 › Hutchinson);
 *   - Hutch++ splits the spectrum into an exact head on an orthonormal basis
 *     Q of Col(O S) and a Hutchinson tail on (I - Q Q^T) (note: 关键设计 ›
 *     Hutch++; summary: Kernmechanisme);
 *   - estimates are summed over layers per sample and the clip factor is
 *     min(C / sqrt(n_i), 1) (note: 方法详解 › 整体框架).
 *
 * Conventions for every entry point
 *   Pointers named A, G, P, S, n, c, head, tail, rank, ws are DEVICE pointers
 *   owned by the caller; the library allocates and frees nothing and keeps no
 *   pointer after returning. Arrays of layer descriptors and trace records are
 *   HOST memory. All work is enqueued on `stream` (0 = the null stream) and
 *   runs asynchronously; results are valid once the stream has been
 *   synchronised. Calls on one stream execute in order, which is what makes
 *   accumulate = 1 a layer sum.
 *   Layouts are row-major and contiguous: A [B][T][d], G [B][T][p],
 *   P [p][k] (or [p][m_t] for the Hutch++ tail), S [p][m_s]; n, c, head,
 *   tail are float [B]; rank is int32 [B]. P and S are shared by the B
 *   samples of a call and drawn by the caller; the library has no RNG, so a
 *   call is a deterministic function of its inputs and is bitwise
 *   reproducible run to run.
 *   Element types: DPNORM_BF16 (A, G, P, S bf16; products accumulate in
 *   fp32) or DPNORM_F32 (all fp32). The widths d and p must be multiples of
 *   8 (bf16) or 4 (fp32) so every row starts on a 16-byte boundary, and base
 *   pointers must be 16-byte aligned. T and B are arbitrary (>= 1).
 *   Workspace: `ws` of at least the size reported by the matching
 *   *_workspace query (256-byte aligned); it may be NULL only when that size
 *   is 0. Concurrent calls on different streams need distinct workspaces.
 *   Errors: every function returns a status and never aborts or prints. The
 *   checks below run on the host before anything is enqueued, so on error no
 *   output has been written. NaN or Inf inside the data is not checked; it
 *   propagates into n and c.
 */
#ifndef DPNORM_H
#define DPNORM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

typedef enum dpnorm_status {
  DPNORM_OK = 0,
  DPNORM_ERR_NULL = 1,        /* a required pointer is NULL */
  DPNORM_ERR_SIZE = 2,        /* a size < 1, too large, misaligned width, bad budget */
  DPNORM_ERR_DTYPE = 3,       /* unknown element type or route */
  DPNORM_ERR_VALUE = 4,       /* C <= 0 or not finite; outputs alias inputs */
  DPNORM_ERR_WORKSPACE = 5,   /* ws_bytes below the workspace query */
  DPNORM_ERR_ALIGN = 6,       /* a base pointer is not 16-byte aligned (ws: 256) */
  DPNORM_ERR_HIP = 7          /* a kernel launch or HIP call failed */
} dpnorm_status;

/* The *_RANGE_MIN_ / *_RANGE_MAX_ enumerators of the two enums callers pass
 * in are range markers, not valid values: they make every int32 a value of
 * the type, so that an unknown value is rejected with DPNORM_ERR_DTYPE
 * instead of being undefined in the library's C++. */
typedef enum dpnorm_dtype {
  DPNORM_F32 = 0,
  DPNORM_BF16 = 1,
  DPNORM_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  DPNORM_DTYPE_RANGE_MAX_ = 2147483647
} dpnorm_dtype;

typedef enum dpnorm_route {
  DPNORM_EXACT_AUTO = 0,      /* explicit when d*p <= T*T, else Gram */
  DPNORM_EXACT_EXPLICIT = 1,  /* sum of squares of A^T G tiles (never stored) */
  DPNORM_EXACT_GRAM = 2,      /* <A A^T, G G^T> over T x T tiles (never stored) */
  DPNORM_ROUTE_RANGE_MIN_ = -2147483647 - 1,
  DPNORM_ROUTE_RANGE_MAX_ = 2147483647
} dpnorm_route;

/* One linear-like layer of a grouped call: device pointers A [B][T][d],
 * G [B][T][p], P [p][k]. */
typedef struct dpnorm_layer {
  const void* A;
  const void* G;
  const void* P;
  int64_t d;
  int64_t p;
} dpnorm_layer;

/* Kernel kinds reported by the traced grouped call. */
typedef enum dpnorm_kernel_kind {
  DPNORM_KERNEL_PREPARE = 1,   /* layer records, work lists, P -> MFMA fragments */
  DPNORM_KERNEL_ROWPROJ = 2,   /* G P (skinny GEMM, streams G) */
  DPNORM_KERNEL_TCONTRACT = 3, /* A^T (G P) + squared Frobenius (streams A) */
  DPNORM_KERNEL_YSUM = 4,      /* split-T partial sums, then squared Frobenius */
  DPNORM_KERNEL_FINISH = 5     /* per-sample sum, layer sum, clip */
} dpnorm_kernel_kind;

/* Event trace for profiling one grouped call. `events` holds `capacity`
 * caller-created events (dpnorm_event_create). The call records events[0]
 * before its first launch and events[j] after its j-th launch, and sets
 * kinds[j-1] to that launch's dpnorm_kernel_kind; `count` returns the number
 * of events recorded. If capacity is too small, DPNORM_ERR_SIZE is returned
 * before anything is enqueued. */
typedef struct dpnorm_trace {
  hipEvent_t* events;
  int32_t* kinds;
  int64_t capacity;
  int64_t count;
} dpnorm_trace;

/* Library version (major * 10000 + minor * 100 + patch). */
int dpnorm_version(void);

/* Human-readable name of a status code (static storage). */
const char* dpnorm_status_string(int status);

/* Hutch++ budget split (note: 关键设计 › Hutch++, and the efficiency table
 * whose Hutch++ FLOP figures correspond to equal column counts): m_s =
 * ceil(k/3) sketch columns (and up to m_s head columns), m_t = k - 2 m_s tail
 * columns. Returns DPNORM_ERR_SIZE when k < 3 (no tail) or k > 96. */
dpnorm_status dpnorm_hutchpp_split(int64_t k, int64_t* m_s, int64_t* m_t);

/* Calibration (not part of the estimator): reads `bytes` (a positive
 * multiple of 16384, at most 2^44) from the device buffer `buf` (16-byte
 * aligned) once, with the direct global-to-LDS loads the stage kernels use,
 * and discards the data. Timing it gives the read rate that load path
 * reaches on this device. Errors: ERR_NULL, ERR_SIZE, ERR_ALIGN, ERR_HIP. */
dpnorm_status dpnorm_read_probe(const void* buf, int64_t bytes, hipStream_t stream);

/* ---- workspace queries (host only; no device work) ---- */
dpnorm_status dpnorm_hutch_workspace(dpnorm_dtype dt, int64_t B, int64_t T, int64_t d, int64_t p,
                                     int64_t k, size_t* bytes);
dpnorm_status dpnorm_hutch_grouped_workspace(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt,
                                             int64_t B, int64_t T, int64_t k, size_t* bytes);
dpnorm_status dpnorm_hutchpp_workspace(dpnorm_dtype dt, int64_t B, int64_t T, int64_t d, int64_t p,
                                       int64_t k, size_t* bytes);
dpnorm_status dpnorm_exact_workspace(dpnorm_dtype dt, int64_t B, int64_t T, int64_t d, int64_t p,
                                     dpnorm_route route, size_t* bytes);

/* Hutchinson estimate of one layer (note: 关键设计 › Hutchinson; summary:
 * Kernmechanisme item 1): n_hat_i = ||A_i^T (G_i P)||_F^2 for every sample,
 * P [p][k] shared by the samples (caller draws N(0, 1/k) entries;
 * 1 <= k <= 64).
 * accumulate = 0 writes n[i] = n_hat_i; accumulate = 1 adds: n[i] += n_hat_i.
 * A, G, P, n device pointers; n must not overlap A, G, P or ws. A bf16 P
 * with k = 16, 32 or 64 that is 16-byte aligned is read in place (one launch
 * fewer than the packed copy other P take; the results are the same). */
dpnorm_status dpnorm_hutch(const void* A, const void* G, const void* P, dpnorm_dtype dt, int64_t B,
                           int64_t T, int64_t d, int64_t p, int64_t k, float* n, int accumulate,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* Hutchinson estimates of L layers summed per sample (note: 方法详解 ›
 * 整体框架, layer sum): n[i] (+)= sum_l ||A_i^(l)T (G_i^(l) P^(l))||_F^2.
 * Same semantics as L dpnorm_hutch calls with accumulate = 1 after the first,
 * in fewer launches. `layers` is a host array of L >= 1 descriptors with
 * device pointers. If c is not NULL, c[i] = min(C / sqrt(n[i]), 1) is also
 * written from the final n (then C must be finite and > 0; c may equal n).
 * Layers whose descriptors carry the same A pointer and the same d (in a
 * transformer block: q, k and v read one input, and so do gate and up) share
 * one pass over A: sum_m ||A^T (G_m P_m)||_F^2 = ||A^T [G_1 P_1 | G_2 P_2 ...]||_F^2,
 * so A is read once for the group (up to 96 projected columns per pass). The
 * result is the same sum, up to rounding order.
 * Workspace: dpnorm_hutch_grouped_workspace given the same descriptors
 * (pointers included) sizes this plan; given NULL A pointers it sizes the
 * plan without sharing, and a call with such a workspace runs without
 * sharing when the shared plan would need more. */
dpnorm_status dpnorm_hutch_grouped(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt, int64_t B,
                                   int64_t T, int64_t k, float* n, int accumulate, float* c, float C,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* dpnorm_hutch_grouped without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Scratch comes from a static device array
 * of DPNORM_STATIC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends; the call itself allocates and frees nothing.
 * The caller still passes every input and output (n, and c when wanted).
 * Arguments, semantics and errors as dpnorm_hutch_grouped, plus:
 *   DPNORM_ERR_WORKSPACE when the call needs more scratch than
 *     DPNORM_STATIC_SCRATCH_BYTES (the size dpnorm_hutch_grouped_workspace
 *     reports for the same descriptors, or for NULL A pointers when sharing
 *     A would not fit); checked before the device is touched;
 *   DPNORM_ERR_VALUE when `stream` belongs to another device than the
 *     current one.
 * All calls on one GPU share its array, and it keeps the last call's
 * contents (nothing in it needs to start at zero): calls that overlap on one
 * GPU, on different streams or host threads, race and must be serialised by
 * the caller. */
#define DPNORM_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
dpnorm_status dpnorm_hutch_grouped_noalloc(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt, int64_t B,
                                           int64_t T, int64_t k, float* n, int accumulate, float* c, float C,
                                           hipStream_t stream);

/* dpnorm_hutch_grouped with an event trace (see dpnorm_trace). */
dpnorm_status dpnorm_hutch_grouped_traced(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt,
                                          int64_t B, int64_t T, int64_t k, float* n, int accumulate,
                                          float* c, float C, void* ws, size_t ws_bytes,
                                          hipStream_t stream, dpnorm_trace* trace);

/* Hutchinson estimate with a +-1 projection stored as bits (note: 实验关键数据
 * › 关键发现 and 局限与展望, which name {-1,+1} 1-bit projections in the
 * style of Achlioptas as the way to shrink P, the memory ceiling at large k;
 * summary: Betekenis en Claims, +-1-valued sketches). The projection is
 * P = S / sqrt(k) with S in {-1,+1}^{p x k} (E[P P^T] = I, as for the
 * N(0, 1/k) matrix), so n_hat_i = ||A_i^T (G_i S)||_F^2 / k.
 * S_bits is a device array [p][ceil(k/32)] of 32-bit words, 4-byte aligned:
 * bit (j % 32) of word (j / 32) of row v is S[v][j], 0 for +1 and 1 for -1
 * (bits past k are ignored); uniformly random words give i.i.d. Rademacher
 * signs. p * ceil(k/32) * 4 bytes instead of p * k * 2 (bf16).
 * The workspace is that of dpnorm_hutch / dpnorm_hutch_grouped with the same
 * sizes. Other arguments, semantics and errors as dpnorm_hutch. The privacy
 * accounting of such projections is outside this library. */
dpnorm_status dpnorm_hutch_sign(const void* A, const void* G, const uint32_t* S_bits, dpnorm_dtype dt,
                                int64_t B, int64_t T, int64_t d, int64_t p, int64_t k, float* n,
                                int accumulate, void* ws, size_t ws_bytes, hipStream_t stream);

/* dpnorm_hutch_grouped with +-1 projections: layers[l].P points to layer l's
 * S_bits as above. Layers sharing A share one pass over it, as there. */
dpnorm_status dpnorm_hutch_sign_grouped(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt,
                                        int64_t B, int64_t T, int64_t k, float* n, int accumulate,
                                        float* c, float C, void* ws, size_t ws_bytes,
                                        hipStream_t stream);

/* Per-layer route between the exact norm and the Hutchinson estimate, summed
 * per sample (note: 实验关键数据 covers full fine-tuning and LoRA; in a LoRA
 * factor one side of W = A^T G is the rank r, far below the p and d of the
 * base layer). A layer whose narrow side min(d, p) is at most k gets its exact
 * norm ||A_i^T G_i||_F^2: contracting W over that side costs no more than a
 * k-column estimate (both read A and G once), so nothing is gained by
 * estimating it. Its P is not read and may be NULL. Every other layer gets
 * the Hutchinson estimate with its P [p][k], as in dpnorm_hutch_grouped.
 * n[i] (+)= sum over layers; c as in dpnorm_hutch_grouped. If routes is not
 * NULL it is a host array of L entries that receives 1 for an exact layer and
 * 0 for an estimated one. Workspace from dpnorm_norms_routed_workspace (same
 * descriptors). Errors as dpnorm_hutch_grouped. */
dpnorm_status dpnorm_norms_routed_workspace(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt,
                                            int64_t B, int64_t T, int64_t k, size_t* bytes);
dpnorm_status dpnorm_norms_routed(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt, int64_t B,
                                  int64_t T, int64_t k, float* n, int accumulate, float* c, float C,
                                  int32_t* routes, void* ws, size_t ws_bytes, hipStream_t stream);

/* Hutch++ estimate of one layer with budget k (note: 关键设计 › Hutch++;
 * summary: Kernmechanisme item 2). With (m_s, m_t) from
 * dpnorm_hutchpp_split(k), S is [p][m_s] (sketch, any scale; N(0,1)
 * suggested) and P is [p][m_t] (tail, entries of variance 1/m_t), both shared
 * by the samples. Per sample:
 *   X = O S with O = G^T A A^T G, formed as G^T (A (A^T (G S)));
 *   Q = orthonormal basis of Col(X) (X formed in fp32), the Q factor of a
 *       Cholesky QR in fp64 with positive diagonal; column j of X is kept
 *       when its residual after projecting out the kept columns before it
 *       (the Cholesky diagonal) exceeds 1e-4 times the largest column norm
 *       of X (rank r_i <= m_s; when O has lower rank than m_s, columns past
 *       it hold only rounding and may still be counted);
 *   head = ||A^T (G Q)||_F^2, tail = ||A^T (G (P - Q Q^T P))||_F^2,
 *   n_hat = head + tail.
 * n (+)= n_hat as for dpnorm_hutch. head, tail (float [B]), rank (int32
 * [B]) and resid (float [B][m_s]) are optional outputs (NULL to skip); they
 * hold this call's values. resid[i][j] is the residual that decided column j
 * of sample i (the Cholesky pivot's square root) over the largest column
 * norm of X_i, so column j is kept iff resid[i][j] > 1e-4 (0 for a zero
 * sketch). The rank is an integer decided on rounded floating point: when
 * O_i has full rank on the sketch (every resid well above 1e-4) it is m_s and
 * matches an exact computation; when O_i has rank below m_s (T, d or p below
 * m_s, or G_i or A_i of low rank) the residuals past that rank hold only the
 * rounding of the fp32 sketch, which can land on either side of 1e-4, so
 * rank may then count some of those columns (the estimate is unaffected:
 * such columns carry rounding-sized parts of O between head and tail).
 * Outputs must not overlap each other, the inputs or ws.
 * k is the total budget, 3 <= k <= 96 (so m_s <= 32 and m_s + m_t <= 64). */
dpnorm_status dpnorm_hutchpp(const void* A, const void* G, const void* S, const void* P, dpnorm_dtype dt,
                             int64_t B, int64_t T, int64_t d, int64_t p, int64_t k, float* n,
                             int accumulate, float* head, float* tail, int32_t* rank, float* resid,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* Exact squared per-sample norm n_i = ||A_i^T G_i||_F^2 (the comparator:
 * note 研究背景与动机 and 相关工作, explicit gradients vs ghost clipping;
 * summary: Complexiteitsreductie). DPNORM_EXACT_EXPLICIT sums squares of
 * A^T G tiles (2 T d p flops per sample); DPNORM_EXACT_GRAM sums the product
 * of A A^T and G G^T tiles (about T^2 (d + p) flops per sample using their
 * symmetry, 2 T^2 (d + p) without); AUTO
 * picks explicit when d*p <= T*T. Nothing of size d x p or T x T is stored.
 * The workspace holds one fp64 partial per tile and sample. */
dpnorm_status dpnorm_exact(const void* A, const void* G, dpnorm_dtype dt, int64_t B, int64_t T, int64_t d,
                           int64_t p, dpnorm_route route, float* n, int accumulate, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* Clip factors (note: 方法详解 › 整体框架): c[i] = min(C / sqrt(n[i]), 1),
 * with n = 0 giving 1, n = +inf giving 0 and NaN propagating. C must be
 * finite and > 0. c == n (in place) is allowed; other overlap is an error. */
dpnorm_status dpnorm_clip_factors(const float* n, int64_t B, float C, float* c, hipStream_t stream);

/* Thin event helpers for profiling (wrap hipEventCreate / Destroy /
 * ElapsedTime / Synchronize); provided so bindings need only this library. */
dpnorm_status dpnorm_event_create(hipEvent_t* ev);
dpnorm_status dpnorm_event_destroy(hipEvent_t ev);
dpnorm_status dpnorm_event_elapsed_ms(hipEvent_t start, hipEvent_t stop, float* ms);
dpnorm_status dpnorm_event_record(hipEvent_t ev, hipStream_t stream);
dpnorm_status dpnorm_event_synchronize(hipEvent_t ev);

#ifdef __cplusplus
}
#endif

#endif /* DPNORM_H */
