/*
 * moe_ragged_bf16.h - C ABI of the deterministic ragged BF16 grouped GEMM for
 * Mixture-of-Experts expert projections, built for AMD MI355X (gfx950).
 *
 * Operations (Cake ragged BF16 grouped GEMM API page, docs.flashinfer.ai,
 * introduction and operations table), for every expert e with rows
 * s_e = offs[e-1] (0 for e == 0) up to t_e = offs[e]:
 *
 *   fwd    Y [s_e:t_e] = X[s_e:t_e] @ W[e]^T        Y  [M, N]    bf16
 *   dgrad  dX[s_e:t_e] = G[s_e:t_e] @ W[e]          dX [M, K]    bf16
 *   wgrad  dW[e]       = G[s_e:t_e]^T @ X[s_e:t_e]  dW [E, N, K] bf16 or fp32
 *
 * with all operands bf16, products summed in fp32 in one fixed order (no atomics),
 * so every output is bitwise identical from run to run on one device with one
 * build.  An expert with no rows gets an exactly-zero (+0.0) dW.  wgrad can
 * instead accumulate into dW (a Megatron-style main_grad), bitwise equal to
 * adding this library's own overwrite dW in dW's dtype (flashinfer PR #8924,
 * "Design and numerics"): fp32, dW[e] = RN32(dW[e] + G_e^T X_e), one IEEE fp32
 * add of the finished product per element; bf16, the bf16 overwrite result is
 * added in bf16: RNE_bf16(RN32(dW[e] + RNE_bf16(G_e^T X_e))).
 *
 * Common conventions of every entry point below:
 *
 *  - Pointers.  Every tensor pointer is a DEVICE pointer on the current HIP
 *    device.  Tensors are dense and row-major: X [m_rows, k], W [E, n, k],
 *    G and Y [m_rows, n], dX [m_rows, k], dW [E, n, k] (k is the unit-stride
 *    dimension of X, W, dX and dW; n of G and Y).  Every tensor pointer must be
 *    16-byte aligned, except offs, which needs 4-byte alignment.  Pointers to
 *    tensors with a row dimension (X, G, Y, dX) may be NULL when m_rows == 0;
 *    all others must be non-NULL.
 *  - Groups.  offs holds num_groups int32 cumulative END offsets, on the device;
 *    the host never reads it.  A caller holding m_indptr[E + 1] (leading zero)
 *    passes m_indptr + 1.  Offsets must be non-decreasing and within
 *    [0, m_rows].  An array that breaks this still accesses no memory out of
 *    bounds: the kernels use end[e] = max over e' <= e of
 *    min(max(offs[e'], 0), m_rows), so it gives the results of that sanitised
 *    array.  Rows at or past end[E-1] belong to no group: fwd and dgrad leave those output rows
 *    untouched and wgrad ignores them.
 *  - Shapes.  1 <= num_groups <= 1024, m_rows >= 0, n >= 8 with n % 8 == 0,
 *    k >= 8 with k % 8 == 0.  (The API page states n % 256 == 0 and k % 64 == 0
 *    for its stable forward entry; here both only need multiples of 8, i.e.
 *    rows of whole 16-byte chunks, the unit of every load and store: the last
 *    256-wide output tile along n or k may be partial, and a reduction over k
 *    (fwd) or n (dgrad) that is not a multiple of 32 ends in a partial stage
 *    whose missing columns load as zeros.)
 *  - Ownership.  The caller owns every buffer.  The library allocates and frees
 *    no device memory, never synchronises the stream or the device, keeps no
 *    pointer after returning and reads no device memory on the host.  Inputs and
 *    outputs must stay alive until the stream has passed the enqueued work.
 *  - Streams.  All work is enqueued on `stream` (a hipStream_t; NULL is the null
 *    stream), in order.  Calls are thread-safe; the only global state is a
 *    per-device property cache filled once.
 *  - Errors.  Every entry returns an mdg_status.  On a validation error nothing
 *    is enqueued and no output is touched.  No exception or abort crosses the
 *    ABI.  A failed kernel launch returns MDG_EHIP.
 */
#ifndef MOE_RAGGED_BF16_H
#define MOE_RAGGED_BF16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Entry points are the library's only exported symbols (it is built with
   hidden visibility by default). */
#if defined(__GNUC__) || defined(__clang__)
#define MDG_API __attribute__((visibility("default")))
#else
#define MDG_API
#endif

#define MDG_ABI_VERSION 6

typedef enum {
  MDG_OK = 0,
  MDG_EINVAL = 1,        /* null pointer, negative size, misaligned pointer, bad enum */
  MDG_EUNSUPPORTED = 2,  /* shape outside the supported set, or device is not gfx950 */
  MDG_EOVERLAP = 3,      /* an output shares a byte with an input, offs or the workspace */
  MDG_EWORKSPACE = 4,    /* workspace missing or smaller than required */
  MDG_EHIP = 5,          /* the HIP runtime reported an error when enqueueing */
  MDG_ENOMEM = 6         /* host memory for a prepared launch could not be allocated */
} mdg_status;

typedef enum { MDG_BF16 = 0, MDG_FP32 = 1 } mdg_dtype;

/* Version of this ABI (MDG_ABI_VERSION of the header the library was built with). */
MDG_API int grouped_det_gemm_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL; an unknown
   code gives "unknown status"). */
MDG_API const char* grouped_det_gemm_status_string(int status);

/*
 * Bytes of device workspace grouped_det_gemm_fwd (resp. _dgrad) needs for these
 * sizes: a small plan table plus fp32 partial tiles of the tail split described
 * below (at most 8 KiB + 64 MiB).  It depends on the sizes only (never on offs or
 * the device).  Returns 0 for invalid sizes.
 */
MDG_API size_t grouped_det_gemm_fwd_workspace_bytes(int64_t m_rows, int64_t n, int64_t k,
                                                    int32_t num_groups);
MDG_API size_t grouped_det_gemm_dgrad_workspace_bytes(int64_t m_rows, int64_t n, int64_t k,
                                                      int32_t num_groups);

/*
 * fwd: Y[s_e:t_e] = X[s_e:t_e] @ W[e]^T  (API page, operations table, "fwd").
 *   x  [m_rows, k] bf16, read.        w [num_groups, n, k] bf16, read.
 *   offs [num_groups] int32, read.    y [m_rows, n] bf16, written (rows of groups only).
 *   workspace: device buffer of at least grouped_det_gemm_fwd_workspace_bytes()
 *      bytes, 256-byte aligned, owned by the caller, contents on entry ignored;
 *      must not overlap any other argument.  Two calls that share a workspace must
 *      be ordered on one stream.
 * Work is scheduled as 256 x 256 output tiles (units).  When the number of units
 * U leaves a remainder T = U mod 256 that would occupy only part of the GPU in
 * the last round, each of those last T units is cut into S consecutive ranges
 * of its reduction (S <= 8, a function of U and the sizes only); each range is
 * summed in fp32 in the one fixed order and a second kernel adds the S partial
 * tiles in range order before rounding to bf16.  Every output is therefore
 * still a fixed function of the inputs: bitwise identical from run to run.
 * m_rows == 0 enqueues nothing.  y must not overlap x, w, offs or the workspace.
 */
MDG_API mdg_status grouped_det_gemm_fwd(const void* x, const void* w, const int32_t* offs, void* y,
                                        int64_t m_rows, int64_t n, int64_t k, int32_t num_groups,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * fwd for callers that cannot allocate device memory at all (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * arguments and results of grouped_det_gemm_fwd, bit for bit, without a
 * workspace argument.  Its scratch (the tail plan and the fp32 partial tiles
 * of the tail split) is a static device array of the library, 64 MiB + 8 KiB,
 * the largest workspace any fwd call needs, so every size grouped_det_gemm_fwd
 * accepts is accepted (a size needing more would get MDG_EWORKSPACE).  Each
 * device the library runs on holds its own copy from the library's loading on
 * that device until the process ends; its address is looked up once per
 * device, at the first call.  No call allocates or frees memory, synchronises
 * or copies; only kernels are enqueued on `stream`.
 * Every call on one device shares that device's array, and nothing in it needs
 * to start cleared: each call writes the plan and partial tiles before reading
 * them, in stream order.  Calls that may overlap on one device (on different
 * streams, or from different threads without ordering) RACE on the array and
 * give undefined results: order them on one stream.
 * m_rows == 0 enqueues nothing.  y must not overlap x, w or offs.
 */
MDG_API mdg_status grouped_det_gemm_fwd_noalloc(const void* x, const void* w, const int32_t* offs, void* y,
                                                int64_t m_rows, int64_t n, int64_t k, int32_t num_groups,
                                                void* stream);

/*
 * dgrad: dX[s_e:t_e] = G[s_e:t_e] @ W[e], W read in place (API page, operations
 * table, "dgrad").
 *   g  [m_rows, n] bf16, read.        w [num_groups, n, k] bf16, read.
 *   offs [num_groups] int32, read.    dx [m_rows, k] bf16, written (rows of groups only).
 *   workspace: as for fwd, of at least grouped_det_gemm_dgrad_workspace_bytes()
 *      bytes; the same tail split applies (the reduction here runs over n).
 * m_rows == 0 enqueues nothing.  dx must not overlap g, w, offs or the workspace.
 */
MDG_API mdg_status grouped_det_gemm_dgrad(const void* g, const void* w, const int32_t* offs, void* dx,
                                          int64_t m_rows, int64_t n, int64_t k, int32_t num_groups,
                                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace grouped_det_gemm_wgrad needs for these sizes: a small
 * work table plus fp32 partial tiles of the fixed-order row split.  It depends
 * on the sizes only (never on offs or the device), so the host can allocate it
 * without a sync.  Returns 0 for invalid sizes.
 */
MDG_API size_t grouped_det_gemm_wgrad_workspace_bytes(int64_t m_rows, int64_t n, int64_t k,
                                                      int32_t num_groups);

/*
 * wgrad: dW[e] = G[s_e:t_e]^T @ X[s_e:t_e]  (API page, operations table, "wgrad";
 * accumulate from flashinfer PR #8924, "Deterministic weight-gradient
 * accumulation" and "Design and numerics").
 *   g [m_rows, n] bf16, read.   x [m_rows, k] bf16, read.   offs [num_groups] int32, read.
 *   dw [num_groups, n, k] of dw_dtype (MDG_BF16 or MDG_FP32):
 *      accumulate == 0: written; an expert with no rows gets +0.0 everywhere.
 *      accumulate != 0: read and written as dw = RN32(dw + dW_e) (MDG_FP32) or
 *        dw = RNE_bf16(RN32(dw + RNE_bf16(dW_e))) (MDG_BF16: both bf16 values
 *        widen exactly, one fp32 add, one rounding).  The add is done for empty
 *        experts too, so -0.0 becomes +0.0 as an add of the zero dW would make
 *        it.  m_rows == 0 then enqueues nothing and leaves dw unchanged.
 *   workspace: device buffer of at least grouped_det_gemm_wgrad_workspace_bytes()
 *      bytes, 256-byte aligned, owned by the caller, contents on entry ignored;
 *      must not overlap any other argument.  Two calls that share a workspace must
 *      be ordered on one stream.
 * The rows of each expert are split into fixed-size consecutive chunks whose
 * size depends only on (m_rows, n, k, num_groups); chunk partials are summed in
 * chunk order by a second kernel on the same stream.  dw must not overlap g, x,
 * offs or the workspace.
 */
MDG_API mdg_status grouped_det_gemm_wgrad(const void* g, const void* x, const int32_t* offs, void* dw,
                                          int dw_dtype, int accumulate,
                                          int64_t m_rows, int64_t n, int64_t k, int32_t num_groups,
                                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Rows per chunk of the wgrad row split for these sizes (a pure function of the
 * sizes; exposed so tests can build cases with and without a split).
 * Returns 0 for invalid sizes.
 */
MDG_API int64_t grouped_det_gemm_wgrad_chunk_rows(int64_t m_rows, int64_t n, int64_t k,
                                                  int32_t num_groups);

/*
 * Zero fill of the rows that belong to no group: out[r, :] = 0 for
 * end <= r < m_rows (Cake ragged BF16 grouped GEMM API page,
 * introduction: groups are consecutive row ranges ending at offs[E-1]; the row
 * padding case of flashinfer PR #8924, "Tests").  fwd and dgrad leave those
 * rows untouched; an autograd wrapper uses this to give them a defined value
 * (zero: they depend on no input) without the host reading offs.
 *   out [m_rows, row_bytes] bytes, row-major, 16-byte aligned; row_bytes a
 *     positive multiple of 16 (at most 2^24).  Written only in the rows named.
 *   offs [num_groups] int32 on the device.  end is the last group end the
 *     GEMM entry points use: the maximum of the offsets clamped to [0, m_rows],
 *     i.e. offs[num_groups-1] for a valid array.  An m_indptr caller passes
 *     m_indptr + 1.
 * m_rows == 0 enqueues nothing.  out must not overlap offs.
 */
MDG_API mdg_status grouped_det_gemm_zero_pad_rows(void* out, const int32_t* offs, int64_t m_rows, int64_t row_bytes,
                                                  int32_t num_groups, void* stream);

/*
 * Prepared launches (Cake ragged BF16 grouped GEMM API page, "Prepared
 * launches": prepare once, launch many times with no allocation and no host
 * synchronisation, capturable into a graph, still valid after new offsets or
 * values are written into the bound buffers).
 *
 * grouped_det_gemm_prepare_{fwd,dgrad,wgrad} take exactly the arguments of the
 * one-shot entry of the same operation (without the stream), run all of its
 * checks and return the same status; on MDG_OK, *launch receives a new
 * host-side object holding the bound pointers and the computed kernel
 * parameters (on any error *launch is set to NULL).  It belongs to the caller,
 * who releases it with grouped_det_gemm_launch_free.  The bound buffers are
 * not copied or owned: they must stay allocated while the launch may be
 * enqueued and until the stream has passed the enqueued work.
 *
 * grouped_det_gemm_launch enqueues the prepared kernels on `stream` (they run
 * exactly as the one-shot entry's would, reading offs and the data on the
 * device at that time): no validation beyond a NULL check and that the current
 * HIP device is the one current at preparation (else MDG_EINVAL), no
 * allocation, no synchronisation and no memset or copy, so it may be called
 * while the stream is being captured into a HIP graph.  Every launch (and
 * every replay of a graph holding one) computes again; an accumulating wgrad
 * adds again.  Launches that share a workspace or an output must be ordered on
 * one stream.  A prepared launch may be used from several threads.
 */
typedef struct mdg_launch mdg_launch;

typedef struct {
  int32_t op;               /* 0 fwd, 1 dgrad, 2 wgrad */
  int32_t device;           /* HIP device of the preparation */
  int32_t kernels;          /* kernels one launch enqueues (0: nothing to do) */
  int32_t gemm_grid;        /* workgroups of the GEMM kernel's persistent grid */
  int32_t dw_dtype;         /* wgrad: MDG_BF16 or MDG_FP32 */
  int32_t accumulate;       /* wgrad: 1 if the launch adds into dw */
  int32_t chunk_rows;       /* wgrad: rows per chunk of the fixed-order row split */
  int32_t tail_slots;       /* fwd/dgrad: fp32 partial tiles available to the tail split */
  int64_t workspace_bytes;  /* workspace bytes the launch uses */
} mdg_launch_info;

MDG_API mdg_status grouped_det_gemm_prepare_fwd(const void* x, const void* w, const int32_t* offs, void* y,
                                                int64_t m_rows, int64_t n, int64_t k, int32_t num_groups,
                                                void* workspace, size_t workspace_bytes, mdg_launch** launch);
MDG_API mdg_status grouped_det_gemm_prepare_dgrad(const void* g, const void* w, const int32_t* offs, void* dx,
                                                  int64_t m_rows, int64_t n, int64_t k, int32_t num_groups,
                                                  void* workspace, size_t workspace_bytes, mdg_launch** launch);
MDG_API mdg_status grouped_det_gemm_prepare_wgrad(const void* g, const void* x, const int32_t* offs, void* dw,
                                                  int dw_dtype, int accumulate,
                                                  int64_t m_rows, int64_t n, int64_t k, int32_t num_groups,
                                                  void* workspace, size_t workspace_bytes, mdg_launch** launch);
MDG_API mdg_status grouped_det_gemm_launch(const mdg_launch* launch, void* stream);
/* Describes a prepared launch (MDG_EINVAL for NULL arguments). */
MDG_API mdg_status grouped_det_gemm_launch_info(const mdg_launch* launch, mdg_launch_info* info);
/* Releases a prepared launch (NULL is ignored).  Work already enqueued is unaffected. */
MDG_API void grouped_det_gemm_launch_free(mdg_launch* launch);

#ifdef __cplusplus
}
#endif

#endif /* MOE_RAGGED_BF16_H */
