/*
 * lq.h -- C ABI of the MI355X (gfx950) int8-state Gated DeltaNet / Kimi Delta
 * Attention decode path ("LeapQuant"): liblq.so.
 *
 * Method sources (web pages about one preprint):
 *   [abstract]  LeapQuant abstract, HFEPX eval-paper page (opentrain.ai),
 *               section "Abstract".
 *   [forum]     zhichai.net forum mirror "LeapQuant: Training-Free 8-bit
 *               Quantization for Linear Attention Recurrent States", section
 *               "Abstract (translated)", techniques 1-3.
 *   [news ¶n]   globaltechnewsdesk.com article "A linear-attention method
 *               cuts state ...", paragraph n.
 *
 * Model.  Per (batch b, head h) the recurrent state is H (dk x dv; row i = key
 * channel, column j = value channel).  One token (q, k in R^dk, v in R^dv,
 * beta, alpha) updates it by the gated delta rule
 *     H <- (I - beta k k^T) D H + beta k v^T,   o = H^T q  (after the update),
 * with D = alpha I (decay_mode LQ_DECAY_SCALAR, Gated DeltaNet) or
 * D = diag(alpha) (LQ_DECAY_PER_KEY, Kimi Delta Attention).
 *
 * Stored state (the "codec"; [news ¶5]: 1.19 bytes per value at
 * dk = dv = 128, C = 4):  H = deq + sum_c e_{idx_c} cv_c^T with
 * deq_ij = sq_ij * row_scale_i * col_scale_j,  sq int8 in [-127, 127].
 * The int8 matrix of a head is dk*dv bytes in the operand order of the int8
 * matrix cores.  Element (i, j) of H's quantized residual (key channel i,
 * value channel j) is byte
 *     off(i, j) = ((((j/16)*KS + i/64)*G + (i%64)/16)*16 + j%16)*16 + i%16,
 * with G = min(4, dk/16) and KS = ceil(dk/64).  16-channel runs of one value
 * column are contiguous, and each 1 KB block is one column tile's operand for
 * one 64-channel K step.  At dk = 16 this is value-column-major (j*dk + i).
 * It stays fixed for a window of W tokens ([news ¶3]); the window's updates
 * live in an fp32 buffer (see lq_gdn_decode_step) and the state is rebuilt
 * and requantized once at the window's end (lq_gdn_window_flush).
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers, owned by the caller, contiguous
 *     row-major in the shapes given, 16-byte aligned, except beta and the
 *     scalar-mode alpha (one float per head), which need 4-byte alignment
 *     only.  The library allocates no device memory, keeps no global state
 *     except the last HIP error code (per thread) and, while kernel timing is
 *     on, its timing records; it never synchronises (except
 *     lq_timing_collect) and the compute entry points are re-entrant.
 *   - `stream` is a hipStream_t (NULL = the default stream); work is enqueued
 *     asynchronously on it.
 *   - Return value: LQ_OK or an LQ_ERR_* code.  Argument checks run first and
 *     make no HIP call; on any error nothing is enqueued.  LQ_ERR_HIP means a
 *     launch failed; lq_last_hip_error() gives the hipError_t.
 *   - Non-finite inputs are not checked; they propagate.
 *   - Supported: dk = dv in {16, 64, 128}; 1 <= W <= 32; 0 <= C <= 8.  The
 *     plain calls take one window position for the whole batch (lockstep);
 *     the *_ragged calls take one per batch row from a device array.
 *   - Token vectors q, k, v and outputs o are fp32 or bf16 (lq_dims.io_dtype);
 *     everything else is fp32 (int8 / int32 where stated).
 *   - Batch rows are independent: rows b0 .. b1-1 of a batch are a batch of
 *     their own (every pointer advanced by b0 rows, lq_dims.B = b1 - b0), and
 *     calls on disjoint row ranges may run at the same time on different
 *     streams.  Each (row, head) is computed the same way whatever the batch
 *     of its call, so the results do not depend on the split.
 */
#ifndef LQ_H
#define LQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum lq_status {
    LQ_OK = 0,
    LQ_ERR_NULL = 1,          /* a required pointer is NULL */
    LQ_ERR_DIMS = 2,          /* B, H, dk, dv, W <= 0; C < 0 or C > dk; bad mode or dtype flag */
    LQ_ERR_UNSUPPORTED = 3,   /* valid but not built: dk/dv, W > 32 or C > 8 */
    LQ_ERR_WINDOW_FULL = 4,   /* decode_step with pos >= W: flush first */
    LQ_ERR_POS = 5,           /* pos < 0, n_buffered outside [0, W], T < 0 */
    LQ_ERR_ALIGN = 6,         /* a pointer is misaligned (see conventions) */
    LQ_ERR_HIP = 7            /* kernel launch failed, see lq_last_hip_error() */
};

enum lq_decay_mode { LQ_DECAY_SCALAR = 0, LQ_DECAY_PER_KEY = 1 };

/* Element type of the token vectors q, k, v and of the outputs o (the gates
 * alpha, beta and everything in lq_state stay fp32).  bf16 values are widened
 * exactly; outputs are rounded to nearest, ties to even. */
enum lq_io_dtype { LQ_IO_F32 = 0, LQ_IO_BF16 = 1 };

/* Problem shape.  smooth: 1 = residual smoothing on (per-column scaling,
 * [forum] technique 3), 0 = off (col_scale written as 1).  io_dtype: an
 * lq_io_dtype. */
typedef struct lq_dims {
    int32_t B, H, dk, dv, W, C;
    int32_t decay_mode;
    int32_t smooth;
    int32_t io_dtype;
} lq_dims;

/* Device arrays of one layer's quantized state and window buffer.
 * gd = dk for LQ_DECAY_PER_KEY, 1 for LQ_DECAY_SCALAR.
 *   sq        int8  [B,H,dk*dv]   quantized residual, byte off(i, j) per head
 *   row_scale fp32  [B,H,dk]      per-row scale (0 for an all-zero row)
 *   col_scale fp32  [B,H,dv]      per-column smoothing factor
 *   comp_idx  int32 [B,H,C]       compensator rows, ascending
 *   comp_val  fp32  [B,H,C,dv]    compensator rows' values (exact fp32)
 *   buf_k     fp32  [B,H,W,dk]    window buffer: keys k_n
 *   buf_m     fp32  [B,H,W,dv]    window buffer: m_n = u_n - Hb^T y_n (see
 *                                 lq_gdn_decode_step)
 *   buf_g     fp32  [B,H,W,gd]    window buffer: window-local cumulative log decay
 * comp_idx/comp_val may be NULL when C = 0. */
typedef struct lq_state {
    int8_t *sq;
    float *row_scale;
    float *col_scale;
    int32_t *comp_idx;
    float *comp_val;
    float *buf_k;
    float *buf_m;
    float *buf_g;
} lq_state;

/*
 * One decode token for every (b, h).  [abstract]: while a window is open the
 * 8-bit state is left as it is and each output also uses the window's updates,
 * kept in full precision; [forum] technique 2: compensator tokens are updated
 * exactly like ordinary tokens.
 *
 * pos = n = number of tokens already buffered in this window (0..W-1).
 * With Hb the window-base state (the dequantized codec, fixed for the
 * window), g_n = g_{n-1} + log alpha (g_{-1} = 0), E_i = exp(g_n - g_i),
 * rr_i = <k, E_i o k_i> and a_i = <q, E_i o k_i> (a_n = <q, k>), the step
 * appends slot n = (k, g_n, m_n),
 *     m_n = beta (v - Hb^T (exp(g_n) o k) - sum_{i<n} rr_i m_i),
 * and writes
 *     o = Hb^T (exp(g_n) o q) + sum_{i<=n} a_i m_i,
 * which is exactly H_n^T q for the state H_n reached from Hb by the window's
 * n+1 delta-rule steps.  (In the WY form of those steps,
 * H_n = A_n Hb + sum_i (E_i o k_i) u_i^T with A_n = Gamma_n - sum_i
 * (E_i o k_i) y_i^T; the buffer keeps m_i = u_i - Hb^T y_i, i.e. the WY
 * factors projected once through the fixed Hb.)
 *   q, k  [B,H,dk];  v, o [B,H,dv]  (fp32 or bf16 per d->io_dtype);  beta fp32 [B,H];
 *   alpha fp32 [B,H] (scalar mode) or [B,H,dk] (per-key mode), in (0, 1].
 * Reads the codec and buffer slots 0..n-1; writes buffer slot n and o.
 * Errors: LQ_ERR_WINDOW_FULL if pos >= W, LQ_ERR_POS if pos < 0.
 */
int lq_gdn_decode_step(const lq_dims *d, const lq_state *st, int32_t pos,
                       const void *q, const void *k, const void *v,
                       const float *alpha, const float *beta, void *o, void *stream);

/*
 * Window boundary for every (b, h) ([news ¶3]: the state is rebuilt and
 * quantized once at the boundary; [forum] techniques 2-3, [news ¶4]).
 * From the codec and n_buffered = N slots (0..W) it rebuilds
 *     H = Gamma Hb + sum_{i<N} (E_{N-1,i} o k_i) m_i^T
 * (Gamma = diag exp(g_{N-1})), then requantizes it in place:
 *   1. m_i = max_j |H_ij|; the C rows with the largest m_i (ties: lower row)
 *      become compensator tokens, comp_idx ascending, comp_val = exact rows;
 *      R = H with those rows zeroed;
 *   2. col_scale_j = max_i |R_ij| (1 if below 2^-120, or if smooth = 0);
 *      Y_ij = R_ij * (1 / col_scale_j);
 *   3. rho_i = max_j |Y_ij|;  row_scale_i = rho_i / 127;
 *      sq_ij = clamp(rint(Y_ij * (127 / rho_i)), -127, 127); a row with
 *      rho_i below 2^-120 is all zeros with row_scale_i = 0;
 * every step one IEEE fp32 operation (round to nearest even), so the bytes
 * are a function of the fp32 H.  h_out (nullable, fp32 [B,H,dk,dv])
 * receives that fp32 H.  n_buffered = 0 is a no-op.  The caller then
 * restarts the window at pos 0.
 * Errors: LQ_ERR_POS if n_buffered < 0 or > W.
 */
int lq_gdn_window_flush(const lq_dims *d, const lq_state *st, int32_t n_buffered,
                        float *h_out, void *stream);

/*
 * lq_gdn_decode_step at position pos followed by lq_gdn_window_flush of
 * pos + 1 slots, in one launch: the usual call for a window's last token
 * (pos = W - 1; [news ¶3]: no update is skipped, and the state is rebuilt and
 * requantized at the boundary).  Same arguments, layouts and effects as the
 * two calls: writes o, buffer slot pos (k, g, m) and the requantized codec,
 * and h_out (nullable) receives the fp32 H of the flush.  The result equals
 * the two calls up to fp32 rounding in o, m_pos and H (the decode's
 * projections Hb^T (exp(g_n) o x) are evaluated as (Gamma Hb)^T x from the
 * flush's fp32 Gamma Hb instead of the int8 matrix cores); the requantized
 * bytes follow the fp32 H written to h_out exactly as in the flush.
 * The caller then restarts the window at pos 0.
 * Errors: LQ_ERR_WINDOW_FULL if pos >= W, LQ_ERR_POS if pos < 0, plus those
 * of the two calls.
 */
int lq_gdn_decode_step_flush(const lq_dims *d, const lq_state *st, int32_t pos,
                             const void *q, const void *k, const void *v,
                             const float *alpha, const float *beta, void *o, float *h_out,
                             void *stream);

/*
 * Ragged windows (sequences of a batch at different window positions, as in
 * serving).  Same as lq_gdn_decode_step, with the position of batch row b
 * read from the DEVICE array pos[b] (int32 [B], 4-byte aligned): every head
 * of row b appends slot pos[b].  A row with pos[b] outside [0, W) is skipped
 * (its o rows and buffer are left untouched).  The caller keeps pos.
 * Errors: as lq_gdn_decode_step (LQ_ERR_NULL / LQ_ERR_ALIGN also for pos).
 */
int lq_gdn_decode_step_ragged(const lq_dims *d, const lq_state *st, const int32_t *pos,
                              const void *q, const void *k, const void *v,
                              const float *alpha, const float *beta, void *o, void *stream);

/*
 * Ragged windows: lq_gdn_window_flush with the number of buffered slots of
 * batch row b read from the DEVICE array n_buffered[b] (int32 [B]).  Rows
 * with n_buffered[b] = 0 (or outside [0, W]) are left untouched, as are their
 * h_out rows.  A row whose window is full (or whose sequence ends) is passed
 * its slot count and restarts at position 0.
 * Errors: as lq_gdn_window_flush (LQ_ERR_NULL / LQ_ERR_ALIGN also for
 * n_buffered).
 */
int lq_gdn_window_flush_ragged(const lq_dims *d, const lq_state *st, const int32_t *n_buffered,
                               float *h_out, void *stream);

/*
 * Ragged windows: lq_gdn_decode_step_flush with the position of batch row b
 * read from the DEVICE array pos[b] (int32 [B], 4-byte aligned): every head
 * of row b decodes its token into slot pos[b] and flushes pos[b] + 1 slots.
 * Rows with pos[b] outside [0, W) are left untouched (codec, buffer, o and
 * h_out rows), so one call serves the rows whose window fills (or whose
 * sequence ends) while lq_gdn_decode_step_ragged serves the others, e.g. on
 * a second stream at the same time: the two calls touch disjoint rows.
 * Errors: as lq_gdn_decode_step_flush (LQ_ERR_NULL / LQ_ERR_ALIGN also for pos).
 */
int lq_gdn_decode_step_flush_ragged(const lq_dims *d, const lq_state *st, const int32_t *pos,
                                    const void *q, const void *k, const void *v,
                                    const float *alpha, const float *beta, void *o, float *h_out,
                                    void *stream);

/*
 * Quantizes an fp32 state h [B,H,dk,dv] into the codec of st (steps 1-3 of
 * lq_gdn_window_flush; buffers untouched).  Used to start decoding from a
 * prefilled state.
 */
int lq_gdn_state_quantize(const lq_dims *d, const float *h, const lq_state *st, void *stream);

/*
 * Checkpoints of the quantized state ([news ¶5]: about 1.19 bytes per value
 * with scales and correction terms), e.g. for prefix caching at window
 * boundaries.  The blob holds one record per head, in (b, h) order (the H
 * records of a sequence are adjacent), each lq_checkpoint_bytes(d) / (B*H)
 * bytes:  sq (dk*dv int8, stored order off(i, j)) | row_scale (4*dk) |
 * col_scale (4*dv) | comp_val (4*C*dv) | comp_idx (4*C) | zero padding to a
 * multiple of 16 bytes.  blob: device memory, 16-byte aligned, caller-owned.
 * Pack reads the codec arrays of st; unpack writes them (the window buffer
 * is not part of a checkpoint: take one right after a flush).
 * Errors: LQ_ERR_NULL, LQ_ERR_ALIGN, LQ_ERR_DIMS, LQ_ERR_UNSUPPORTED.
 */
size_t lq_checkpoint_bytes(const lq_dims *d);
int lq_gdn_state_pack(const lq_dims *d, const lq_state *st, void *blob, void *stream);
int lq_gdn_state_unpack(const lq_dims *d, const void *blob, const lq_state *st, void *stream);

/*
 * Writes the fp32 state the codec stands for into h_out [B,H,dk,dv]
 * (row-major): (sq_ij * row_scale_i) * col_scale_j, plus comp_val on the
 * compensator rows.
 */
int lq_gdn_state_dequantize(const lq_dims *d, const lq_state *st, float *h_out, void *stream);

/*
 * Dense fp32-state gated delta rule over T tokens, state h [B,H,dk,dv] updated
 * in place.  The fp32-state baseline the pages compare against ([abstract]:
 * FP32 baseline), and the prefill that produces a starting state.  Inputs are
 * [T,B,H,...] (shapes as in lq_gdn_decode_step); o (nullable) [T,B,H,dv].
 * d->W, d->C and d->smooth are ignored.  Errors: LQ_ERR_POS if T < 0.
 */
int lq_gdn_fp32_recurrence(const lq_dims *d, float *h, int32_t T,
                           const void *q, const void *k, const void *v,
                           const float *alpha, const float *beta, void *o, void *stream);

/*
 * Prefill of a prompt: the state after T tokens, computed in fp32 in chunks
 * of 16 tokens (the chunk form of the same recurrence: within a chunk the
 * updates are combined in WY form and applied with fp32 matrix-core
 * products), then quantized once into st's codec (steps 1-3 of
 * lq_gdn_window_flush).  [abstract]: decoding reads the low-bit state;
 * [news ¶3]: it is quantized once per window, not per token, so the prompt
 * runs in fp32 and only its final state is quantized.
 *   h      fp32 [B,H,dk,dv] (row-major), in: the state before the prompt
 *          (zeros for a new sequence), out: the state after it;
 *   q..beta as lq_gdn_fp32_recurrence, [T,B,H,...];
 *   o      nullable fp32 [T,B,H,dv]: every prompt token's output;
 *   st     nullable: codec arrays written (buffers untouched); NULL leaves
 *          the state in fp32 only.
 * T = 0 only quantizes h.  The results equal lq_gdn_fp32_recurrence followed
 * by lq_gdn_state_quantize up to fp32 rounding in h and o; the codec bytes
 * are those of the fp32 h written.
 * Errors: LQ_ERR_POS if T < 0; LQ_ERR_NULL / LQ_ERR_ALIGN for h and the
 * token arrays.
 */
int lq_gdn_prefill(const lq_dims *d, const lq_state *st, float *h, int32_t T,
                   const void *q, const void *k, const void *v,
                   const float *alpha, const float *beta, void *o, void *stream);

/* Bytes of one layer's codec arrays (sq, scales, compensators), i.e.
 * B*H*(dk*dv + 4dk + 4dv + C*(4dv + 4)); 0 if d is NULL or invalid. */
size_t lq_state_bytes(const lq_dims *d);

/* Bytes of one layer's window buffer (buf_k, buf_m, buf_g), i.e.
 * B*H*W*4*(dk + dv + gd); 0 if invalid. */
size_t lq_buffer_bytes(const lq_dims *d);

/* Static description of a status code (never NULL). */
const char *lq_status_str(int status);

/* hipError_t of the last LQ_ERR_HIP returned on the calling thread (0 if none). */
int lq_last_hip_error(void);

/* LQ_OK if every entry point accepts the shape d (same checks they run). */
int lq_check_dims(const lq_dims *d);

/*
 * Kernel timing (measurement support, not part of the method).  While
 * enabled, every kernel the library launches carries a start/stop event pair
 * that records the kernel's own execution interval (hipExtLaunchKernelGGL),
 * so the durations exclude launch gaps and host overhead.  Kernel families:
 */
enum {
    LQ_KERNEL_DECODE = 0,       /* lq_gdn_decode_step */
    LQ_KERNEL_FLUSH = 1,        /* lq_gdn_window_flush */
    LQ_KERNEL_QUANTIZE = 2,     /* lq_gdn_state_quantize */
    LQ_KERNEL_DEQUANTIZE = 3,   /* lq_gdn_state_dequantize */
    LQ_KERNEL_FP32_RECURRENCE = 4,
    LQ_KERNEL_CHECKPOINT = 5,   /* lq_gdn_state_pack / lq_gdn_state_unpack */
    LQ_KERNEL_DECODE_FLUSH = 6, /* lq_gdn_decode_step_flush */
    LQ_KERNEL_PREFILL = 7,      /* lq_gdn_prefill (its quantization: LQ_KERNEL_QUANTIZE) */
    LQ_KERNEL_MEASURE = 8       /* lq_measure_stream_read */
};

/* on = 1: drop earlier records and start recording (at most 65536 launches;
 * later ones run untimed); on = 0: stop recording.  Process-wide; not for
 * concurrent use from several host threads. */
int lq_timing_enable(int32_t on);

/* Waits for the recorded launches, writes the first min(max_records, n) of
 * them in launch order (family[i], ms[i] = kernel duration in milliseconds;
 * host arrays, may be NULL if max_records = 0), sets *count = n and drops the
 * records.  Errors: LQ_ERR_NULL, LQ_ERR_HIP. */
int lq_timing_collect(int32_t max_records, int32_t *family, float *ms, int32_t *count);

/*
 * Streaming-read reference (measurement support, not part of the method):
 * what a bare read of a launch's bytes costs on the GPU at hand, the ceiling
 * for a kernel of the same launch shape.  Reads n_slices slices of
 * slice_bytes contiguous bytes each from src (n_slices * slice_bytes bytes in
 * all, non-temporal 16-byte loads) and writes write_bytes bytes per slice to
 * sink (the XOR of the slice's 16-byte pieces, so no load is dead).
 *   mode 0: one 256-lane workgroup per slice, every load issued before any
 *           is used (the shape of a decode launch: one workgroup per head);
 *   mode 1: `grid` workgroups walking the slices in grid stride.
 * src, sink: device, 16-byte aligned; slice_bytes a multiple of 16 in
 * [16, 65536]; write_bytes a multiple of 16 in [0, 4096] (sink may be NULL
 * when it is 0), sink holds n_slices * write_bytes bytes; n_slices >= 1;
 * grid >= 1 (mode 1 only).  Timed like the other kernels
 * (LQ_KERNEL_MEASURE).
 * Errors: LQ_ERR_NULL, LQ_ERR_ALIGN, LQ_ERR_DIMS (a size out of range or a
 * bad mode).
 */
int lq_measure_stream_read(const void *src, size_t slice_bytes, int32_t n_slices, int32_t mode,
                           int32_t grid, void *sink, size_t write_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LQ_H */
