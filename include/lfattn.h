/*
 * lfattn: band + global sparse self-attention, forward pass, on AMD MI355X
 * (gfx950).  C ABI.
 *
 * Operation (per batch b, head h, query row i; Q, K, V, O are [B, H, N, D]):
 *
 *   S_i = { 0, ..., N-1 }                                        if i in G
 *   S_i = { i + d_h*k : -hw <= k <= hw, 0 <= i + d_h*k < N }  u  G  otherwise
 *   O_i = sum_{j in S_i} softmax_j(scale * Q_i . K_j) V_j
 *
 * with hw = floor(window / 2), d_h the dilation of head h and G the set of
 * global token positions.  This is attention as in Eq. (1) of "Unlimiformer:
 * Long-Range Transformers with Unlimited Length Input" (section 2.3)
 * restricted to the Longformer pattern of the Ultralytics glossary page
 * "Longformer" (section on how the attention works: the sliding-window,
 * dilated-window and global-attention bullets, and the mask sample there,
 * which uses |i - j| <= window // 2 and sets a global token's whole row and
 * column).  GMAT's memory tokens ("GMAT: Global Memory Augmentation for
 * Transformers", section "Global Memory") are the case G = {0, ..., M-1} with
 * the main sequence after them.  The page gives no formula for dilation; this
 * library reads it as "the same 2*hw+1 offsets, spaced d_h apart".  A global
 * key that already lies in a row's band is scored once (set union).
 *
 * Two generalisations, both from the same glossary section: G may differ
 * between batch elements (G_b; the page's closing paragraph notes that the
 * Hugging Face implementation takes the global tokens as a per-sequence
 * global_attention_mask), and the global rows may have their own projections
 * (the global-attention bullet: global attention uses separate query, key and
 * value projections).  The page does not say which scores those enter; this
 * library reads them as the global rows' own attention:
 *
 *   O_i = sum_{j < N} softmax_j(scale * Qg_i . Kg_j) Vg_j        if i in G_b
 *
 * while every other row keeps Q, K, V for its band and for the global keys.
 *
 * A causal variant (lfattn_create_causal) keeps the band's left half and the
 * row itself, S_i = { i + d_h*k : -hw <= k <= 0, i + d_h*k >= 0 }, with no
 * global tokens: the dilated-window bullet's use case is a character-level
 * language model, which predicts each character from the ones before it (the
 * page states no causal rule; this is the reading taken).
 *
 * A chunked variant (lfattn_create_chunked) is GMAT's C x k chunked
 * self-attention with M memory tokens ("GMAT: Global Memory Augmentation for
 * Transformers", sections "Global Memory" and "Chunked self-attention"): the
 * memory is positions 0 .. M-1 (G = {0, ..., M-1}); the main sequence after it
 * is cut into contiguous chunks of C positions (the last one shorter when
 * N - M is not a multiple of C), and a main row scores its own chunk and the
 * memory, S_i = {0, ..., M-1} u {c0, ..., min(c0 + C, N) - 1} with
 * c0 = M + C * floor((i - M) / C).  Memory rows score all N keys.
 *
 * Layouts.  Q, K, V, O: contiguous [B, H, N, D] arrays in device memory, D
 * fastest, 16-byte aligned, element type set at create (float, or bfloat16
 * stored as 16-bit words).  Accumulation is always fp32; bf16 outputs are
 * rounded to nearest even.
 *
 * Ownership.  Q, K, V, O (and Qg, Kg, Vg) belong to the caller.  The inputs
 * are only read; O is fully overwritten and must not overlap any input.  The
 * host arrays passed to the create calls (dilation, global_idx, global_mask)
 * are copied; the caller may free them on return.  The handle owns its
 * device tables and workspace and frees them in lfattn_destroy.
 *
 * Execution.  The forward calls allocate nothing and do not wait on the host:
 * it enqueues its kernels on the given HIP stream and returns.  Device-side
 * errors surface at the caller's next synchronisation, as for any HIP call.
 * A handle keeps per-call workspace, so one handle must not be used by two
 * forwards that may run at the same time (e.g. on two streams); create one
 * handle per stream instead.  All calls on a handle must be made with the
 * device that was current at lfattn_create.
 *
 * Tuning.  bf16 handles run the band work in 64-row workgroups (the keys of
 * each split in two halves) or 128-row ones (one key stream shared by four
 * 32-row blocks), chosen at lfattn_create from the number of row blocks and
 * the device's compute units.  The environment variable LFATTN_BAND_ROWS,
 * set to 64 or 128 when lfattn_create runs, overrides that choice; results
 * are the same either way up to floating-point summation order.  The
 * backward (bf16) takes 64-row items with split key tiles on its query side
 * and 64-key items with split row tiles on its key side; LFATTN_BWD_ROWS, 64
 * or 128 when lfattn_create runs, sets both sides to that size.  At D = 64
 * its query side runs three or four wavefronts per SIMD (four when its items
 * come to two or more rounds of the three-per-CU slots);
 * LFATTN_BWD_ROWS_WPE, 3 or 4, overrides that choice (the same results).  With
 * LFATTN_FUSE_MERGE=1 at lfattn_create, bf16 handles merge the global rows'
 * partial results inside the band launch instead of a separate launch (the
 * same results; slower on the workloads measured, hence not the default).
 *
 * Errors.  Every entry point returns a status synchronously.  Arguments are
 * checked before any HIP call is made, so invalid arguments never touch the
 * device.
 */
#ifndef LFATTN_H
#define LFATTN_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lfattn_ctx* lfattn_t;

typedef enum {
  LFATTN_OK = 0,
  LFATTN_EINVAL = 1,      /* bad argument: null/misaligned pointer, size, window,
                             dilation, global index outside [0, N), overlap */
  LFATTN_EUNSUPPORTED = 2, /* valid but not implemented: D not 64 or 128, N >= 2^29,
                             or more than 512 distinct global positions with bf16 */
  LFATTN_ENOMEM = 3,      /* device or host allocation failed */
  LFATTN_EHIP = 4,        /* a HIP runtime call or kernel launch failed */
  LFATTN_ESCRATCH = 5     /* lfattn_forward_noalloc: the handle's global-row partials
                             need more than the library's static scratch array */
} lfattn_status;

typedef enum { LFATTN_F32 = 0, LFATTN_BF16 = 1 } lfattn_dtype;

/*
 * Create a handle for one problem shape and pattern.
 *   out        receives the handle (set to NULL on failure).
 *   B, H, N    batch, heads, sequence length (each >= 1).
 *   D          head dimension: 64 or 128.
 *   dtype      element type of Q, K, V and O.
 *   window     >= 0; half-width hw = window / 2 (floor), as in the Longformer
 *              page's sample (window 512 means 256 on each side, inclusive).
 *   dilation   H host ints >= 1, or NULL for all 1 (dilated-window bullet).
 *   global_idx n_global host ints in [0, N), any order, repeats allowed (a
 *              position listed twice is global once); NULL if n_global == 0.
 *              bf16 handles take at most 512 distinct positions.
 *   scale      softmax scale; <= 0 selects 1/sqrt(D) (Eq. (1) of the
 *              Unlimiformer page).  NaN or infinity is EINVAL.
 * Allocates the handle's device tables and workspace on the current device
 * (the only host-to-device copies the library makes happen here).
 */
lfattn_status lfattn_create(lfattn_t* out, int B, int H, int N, int D, lfattn_dtype dtype,
                            int window, const int* dilation, const int* global_idx,
                            int n_global, float scale);

/*
 * As lfattn_create, with one global set per batch element given as a host
 * byte mask: global_mask[b * N + i] nonzero makes position i global in batch
 * element b (the global_attention_mask form the Longformer glossary page's
 * closing paragraph mentions).  NULL: no global positions.  The mask is read
 * during the call only.  bf16 handles take at most 512 global positions per
 * batch element (EUNSUPPORTED beyond).
 */
lfattn_status lfattn_create_masked(lfattn_t* out, int B, int H, int N, int D,
                                   lfattn_dtype dtype, int window, const int* dilation,
                                   const unsigned char* global_mask, float scale);

/*
 * As lfattn_create for the causal band (see the operation above): no global
 * tokens, every row scores itself and the hw keys of its band before it.
 */
lfattn_status lfattn_create_causal(lfattn_t* out, int B, int H, int N, int D,
                                   lfattn_dtype dtype, int window, const int* dilation,
                                   float scale);

/*
 * As lfattn_create for GMAT's chunked attention (see the operation above):
 * chunk >= 1 keys per chunk, 0 <= n_memory <= N memory positions at the start
 * (bf16: n_memory <= 512).  Dilation is 1.  lfattn_forward_global_proj gives
 * the memory rows their own projections, as for any global rows.
 */
lfattn_status lfattn_create_chunked(lfattn_t* out, int B, int H, int N, int D,
                                    lfattn_dtype dtype, int chunk, int n_memory, float scale);

/*
 * Enqueue one forward pass on `stream` (NULL: the null stream).
 * Q, K, V: device pointers to [B, H, N, D] inputs; O: device pointer to the
 * [B, H, N, D] output.  Returns EINVAL for a null or misaligned pointer or an
 * O that overlaps an input, EHIP if a launch fails.
 */
lfattn_status lfattn_forward(lfattn_t ctx, const void* Q, const void* K, const void* V,
                             void* O, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as lfattn_forward, with the global rows' per-chunk partial records
 * kept in the library's static device array (32 MiB per GPU, held until the
 * process ends) instead of the handle's workspace.  Allocates nothing and
 * calls no allocating routine; launches kernels only.  Every call on one GPU
 * shares that GPU's array: two calls that may overlap on one GPU (any
 * streams, any handles) race and must not be made.  Each call writes every
 * record it reads, so the array needs no clearing between calls.  Returns
 * ESCRATCH when the handle's records exceed the array (B * H * ceil(|G| /
 * rows per set) * key chunks * rows per set * (D + 4) * 4 bytes; the
 * 65536-token, 64-global workload needs about 69 MB), EHIP when the array's
 * device address could not be obtained at lfattn_create, otherwise errors as
 * lfattn_forward.
 */
lfattn_status lfattn_forward_noalloc(lfattn_t ctx, const void* Q, const void* K, const void* V,
                                     void* O, hipStream_t stream);

/*
 * Forward pass in which the global rows take their own projections (the
 * global-attention bullet of the Longformer glossary page; see the operation
 * above).  Qg, Kg, Vg: device pointers to [B, H, N, D] arrays laid out like Q
 * (only Qg's global rows are read; Kg and Vg are read at every position); each
 * may be NULL to use Q, K or V instead.  Every row outside its batch element's
 * global set reads only Q, K and V.  lfattn_forward(ctx, Q, K, V, O, s) is this
 * call with Qg = Kg = Vg = NULL.  Errors as lfattn_forward, checked over all
 * seven pointers (O must overlap none of the six inputs).
 */
lfattn_status lfattn_forward_global_proj(lfattn_t ctx, const void* Q, const void* K,
                                         const void* V, const void* Qg, const void* Kg,
                                         const void* Vg, void* O, hipStream_t stream);

/*
 * As lfattn_forward, also writing LSE[b, h, i] = log sum_{j in S_i}
 * exp(scale * Q_i . K_j) (natural log, fp32, [B, H, N] device array that must
 * overlap no other argument), the per-row statistic a backward pass needs.
 * bf16 handles only (EUNSUPPORTED otherwise).
 */
lfattn_status lfattn_forward_lse(lfattn_t ctx, const void* Q, const void* K, const void* V,
                                 void* O, float* LSE, hipStream_t stream);

/*
 * As lfattn_forward_global_proj, also writing LSE as lfattn_forward_lse does
 * (the global rows' from their own projections): the forward whose output
 * and log-sum-exp lfattn_backward_global_proj takes.  bf16 handles only.
 */
lfattn_status lfattn_forward_global_proj_lse(lfattn_t ctx, const void* Q, const void* K,
                                             const void* V, const void* Qg, const void* Kg,
                                             const void* Vg, void* O, float* LSE,
                                             hipStream_t stream);

/*
 * Backward pass: gradients of the forward (lfattn_forward / lfattn_forward_lse,
 * the ordinary projections) for the upstream gradient dO.  Q, K, V: the
 * forward's inputs; O and LSE: its output and log-sum-exp (from
 * lfattn_forward_lse); dO: [B, H, N, D] like O.  Writes dQ, dK, dV: fp32
 * [B, H, N, D] device arrays, fully overwritten, overlapping no input and
 * each other.  With P the forward's weights over each row's key set S_i (the
 * chain rule through the row softmax of Eq. (1) of the Unlimiformer page):
 *   dS_ij = P_ij (dO_i . V_j - dO_i . O_i),   dQ_i = scale sum_j dS_ij K_j,
 *   dK_j = scale sum_i dS_ij Q_i,            dV_j = sum_i P_ij dO_i.
 * bf16 handles (D = 64 or 128; EUNSUPPORTED for fp32), every pattern.
 * Allocates nothing; the handle's workspace holds dO . O per row and the
 * global rows' and keys' partial gradients per key (row) chunk, summed in a
 * fixed order: results are the same bits on every run.  Launches kernels
 * only, so the call may be captured into a HIP graph.
 */
lfattn_status lfattn_backward(lfattn_t ctx, const void* Q, const void* K, const void* V,
                              const void* O, const void* dO, const float* LSE, float* dQ,
                              float* dK, float* dV, hipStream_t stream);

/*
 * Backward pass of the forward with separate global-row projections
 * (lfattn_forward_global_proj_lse; Qg, Kg, Vg may each be NULL for Q, K, V):
 * a global row i of batch element b scores every key with Qg_i, Kg, Vg, so
 * its terms of the chain rule above go to dQg_i, dKg_j, dVg_j, while every
 * other row's go to dQ, dK, dV as in lfattn_backward (the global-attention
 * bullet of the Longformer glossary page: global attention has its own query,
 * key and value projections).  All six outputs are fp32 [B, H, N, D] arrays,
 * fully overwritten (dQ is zero on global rows and dQg on the others),
 * overlapping no input and each other.  With Qg = Q, Kg = K and Vg = V the
 * sums dQ + dQg, dK + dKg and dV + dVg are lfattn_backward's gradients.
 * Errors and execution as lfattn_backward.
 */
lfattn_status lfattn_backward_global_proj(lfattn_t ctx, const void* Q, const void* K,
                                          const void* V, const void* Qg, const void* Kg,
                                          const void* Vg, const void* O, const void* dO,
                                          const float* LSE, float* dQ, float* dK, float* dV,
                                          float* dQg, float* dKg, float* dVg,
                                          hipStream_t stream);

/* Release the handle and its device memory.  The memory is returned with
 * stream-ordered frees behind the work enqueued so far on the stream of the
 * handle's latest call, which must still exist; the host waits for neither
 * that work nor other streams' (on a device without memory pools, the
 * runtime's hipFree waits for the device).  Work that used the handle on
 * other streams must be complete, or ordered before that stream's current
 * point, and every HIP graph that replays captured calls must have finished.
 * NULL is accepted and ignored. */
lfattn_status lfattn_destroy(lfattn_t ctx);

/* Static English text for a status code. */
const char* lfattn_status_string(lfattn_status status);

/*
 * Number of (query, key) pairs one forward scores, summed over B, H and N:
 * sum_i |S_i|, the count the Longformer page's sample takes with mask.sum().
 */
lfattn_status lfattn_scored_pairs(lfattn_t ctx, long long* pairs);

/*
 * Number of (query, key) pairs the band kernel launch scores per forward: the
 * pairs of the rows not in G, plus those of the global rows where the band
 * launch also computes them (bf16; with fp32 a separate kernel
 * does).  The figure a per-kernel throughput is computed from.
 */
lfattn_status lfattn_band_launch_pairs(lfattn_t ctx, long long* pairs);

/*
 * Rows per workgroup of the handle's band launch (*rows: 64 or 128; see
 * Tuning above).  EINVAL for a null argument.
 */
lfattn_status lfattn_band_rows(lfattn_t ctx, int* rows);

/*
 * The canonical global list the handle uses: sorted, without repeats (batch
 * element 0's, for a handle from lfattn_create_masked).  Writes
 * min(n, capacity) positions to out (may be NULL when capacity is 0) and the
 * full count n to *n_out.
 */
lfattn_status lfattn_global_list(lfattn_t ctx, int* out, int capacity, int* n_out);

/* The global list of batch element b (0 <= b < B, else EINVAL), as
 * lfattn_global_list. */
lfattn_status lfattn_global_list_batch(lfattn_t ctx, int b, int* out, int capacity,
                                       int* n_out);

/*
 * Per-kernel timing with HIP events, for measurement.  While enabled, each
 * forward launches its kernels with start and stop events that take each
 * kernel's own begin and end timestamps (at most 4096 forwards are recorded;
 * later ones run untimed).  lfattn_read_timing waits for the recorded events
 * and returns, summed over the recorded forwards, the milliseconds of the band
 * kernel and of the global-row kernels (0 without global positions): the
 * partial and merge kernels, or only the merge where the band launch also
 * computes the global rows' partials (bf16).  Also the number of
 * forwards recorded; then clears the record.
 * Enabling or disabling also clears it.
 */
lfattn_status lfattn_set_timing(lfattn_t ctx, int enable);
lfattn_status lfattn_read_timing(lfattn_t ctx, double* band_ms, double* global_ms,
                                 int* n_forwards);

/*
 * The same for lfattn_backward calls while timing is enabled (at most 1024
 * recorded): the milliseconds, summed over the recorded calls, of the
 * query-side kernel (dQ and the row terms Delta), of the key-side kernel
 * (dK, dV) and of the merge of the global rows' and keys' partial gradients
 * (0 without global positions); the number of calls recorded; then clears
 * that record.
 */
lfattn_status lfattn_read_backward_timing(lfattn_t ctx, double* rows_ms, double* keys_ms,
                                          double* merge_ms, int* n_backwards);

#ifdef __cplusplus
}
#endif

#endif /* LFATTN_H */
