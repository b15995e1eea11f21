/*
 * gdn.h -- C ABI of libgdn.so, a Gated DeltaNet (GDN) token-mixing layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (sources: "Implement the Qwen3.8 Flash Next Rust and Metal text
 * core", DS4Server issue #95, section Implementation and its implementation
 * comment; "Add a performance-parity Qwen3.8-27B Q4 and Q8 text backend on
 * Metal", DS4Server issue #88, section Scope):
 *
 *   1. causal depthwise Conv1D of width W=4 over the concatenated q/k/v input
 *      channels, with a rolling history of the last W-1 inputs, then SiLU;
 *   2. L2 normalisation of every q and k head, x / sqrt(sum x^2 + l2_eps),
 *      q further multiplied by q_scale;
 *   3. the gated delta rule with an fp32 recurrent state per value head
 *      (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025):
 *        S_t = a_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *        o_t = S_t q_t,   a_t = exp(g_t);
 *   4. a sigmoid output gate, y_t = o_t * sigmoid(z_t).
 *
 * One semantic interface with a separately tuned chunked prefill and a
 * single-token decode; the recurrent and conv state are caller-owned buffers
 * kept apart from any attention KV cache (issue #88, section Scope).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - C_ch = 2*H_k*d_k + H_v*d_v input channels, ordered [q | k | v], each part
 *    head-major with the head dimension fastest.  Value head h reads key head
 *    h / (H_v / H_k).
 *  - Layouts are dense and row-major:
 *      x          [B][T][C_ch]        in_dtype
 *      z          [B][T][H_v][d_v]    in_dtype
 *      g, beta    [B][T][H_v]         fp32 (log decay g <= 0, 0 <= beta <= 1)
 *      conv_w     [C_ch][W]           in_dtype; tap W-1 meets the current token
 *      conv_state [B][W-1][C_ch]      in_dtype; oldest row first
 *      rec_state  [B][H_v][d_v][d_k]  fp32; o = S q
 *      y          [B][T][H_v][d_v]    out_dtype
 *  - Device pointers are device memory of the current HIP device, aligned to
 *    their element size; rec_state, the workspaces, and the prefill x, z and
 *    conv_state 16-byte aligned (every token offset of a 16-byte aligned x
 *    stays 16-byte aligned).  The
 *    caller owns every buffer; the library allocates nothing,
 *    keeps no state between calls and is safe to call from several threads
 *    (apart from gdn_prefill_varlen's auxiliary streams and the fixed
 *    scratch of gdn_decode_step_noalloc, each described there).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Compute calls
 *    only enqueue work and never synchronise; save/restore return after the
 *    copy has completed.
 *  - conv_state and rec_state are updated in place.  Outputs and workspace
 *    must not overlap any input or state buffer.
 *  - z may be NULL in every layer call: y is then the ungated readout
 *    o_t = S_t q_t (for a caller that applies its own epilogue, such as
 *    gdn_gated_rmsnorm below).
 *  - Every argument is validated before anything is enqueued; on any error
 *    no caller byte has changed (fail before partial execution: issue #95,
 *    implementation comment).  Values are not checked on the device: inputs
 *    must be finite, g <= 0 and 0 <= beta <= 1.  Errors of work already
 *    enqueued surface when the caller synchronises the stream.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 1

/* Exported from libgdn.so (the library is built with hidden visibility). */
#if defined(__GNUC__)
#define GDN_API __attribute__((visibility("default")))
#else
#define GDN_API
#endif

/* Status codes: 0 on success, negative on error. */
#define GDN_OK 0
#define GDN_ERR_INVALID_ARG (-1)   /* null pointer, bad size or value        */
#define GDN_ERR_UNSUPPORTED (-2)   /* ABI mismatch or geometry not built     */
#define GDN_ERR_ALIGNMENT (-3)     /* device pointer misaligned              */
#define GDN_ERR_ALIAS (-4)         /* output/workspace overlaps an input     */
#define GDN_ERR_WORKSPACE (-5)     /* workspace smaller than required        */
#define GDN_ERR_BLOB_MAGIC (-6)    /* state blob: wrong magic                */
#define GDN_ERR_BLOB_VERSION (-7)  /* state blob: unknown format version     */
#define GDN_ERR_BLOB_SHAPE (-8)    /* state blob: dims or dtype differ       */
#define GDN_ERR_BLOB_SIZE (-9)     /* state blob: buffer size mismatch       */
#define GDN_ERR_BLOB_CHECKSUM (-10) /* state blob: header or payload corrupt */
#define GDN_ERR_HIP (-11)          /* HIP runtime error; see gdn_last_hip_error */
#define GDN_ERR_TOO_LARGE (-12)    /* beyond the fixed scratch of gdn_decode_step_noalloc */

/* Element types.  GDN_F16 is an output type only (y). */
#define GDN_F32 0
#define GDN_BF16 1
#define GDN_F16 2

/* Geometry and numeric options, passed by pointer to every call.
 * Built geometries: d_k = d_v in {16, 128}, W = 4, H_v a multiple of H_k,
 * in_dtype in {GDN_F32, GDN_BF16}, out_dtype in {GDN_F32, GDN_BF16, GDN_F16},
 * l2_eps >= 0. */
typedef struct gdn_dims {
  int32_t abi;       /* must be GDN_ABI_VERSION                     */
  int32_t B;         /* sequences                                    */
  int32_t H_k, H_v;  /* key heads, value heads                       */
  int32_t d_k, d_v;  /* head dimensions                              */
  int32_t W;         /* conv taps                                    */
  int32_t in_dtype;  /* x, z, conv_w, conv_state                     */
  int32_t out_dtype; /* y (GDN_F16 allowed)                          */
  float l2_eps;      /* epsilon inside the root of the L2 norm       */
  float q_scale;     /* extra factor on normalised q                 */
} gdn_dims;

/* ABI version compiled into the library (equals GDN_ABI_VERSION). */
GDN_API int gdn_abi_version(void);

/* Static text for a status code. Never NULL. */
GDN_API const char *gdn_status_str(int status);

/* Text of the last GDN_ERR_HIP raised on the calling thread ("" if none). */
GDN_API const char *gdn_last_hip_error(void);

/* Buffer sizes in bytes; 0 when `dims` is invalid.
 *   rec_state:  B*H_v*d_v*d_k*4
 *   conv_state: B*(W-1)*C_ch*sizeof(in_dtype)
 *   state blob: header + conv_state + rec_state bytes (see gdn_state_save) */
GDN_API size_t gdn_rec_state_bytes(const gdn_dims *dims);
GDN_API size_t gdn_conv_state_bytes(const gdn_dims *dims);
GDN_API size_t gdn_state_blob_bytes(const gdn_dims *dims);

/* Workspace needed by gdn_prefill_chunked for T tokens in chunks of `chunk`
 * tokens, and by gdn_decode_step.  0 when the arguments are invalid. */
GDN_API size_t gdn_prefill_workspace_bytes(const gdn_dims *dims, int64_t T, int32_t chunk);
GDN_API size_t gdn_decode_workspace_bytes(const gdn_dims *dims);

/* Steps 1-2 alone over T >= 1 tokens (issue #88, section Measurements and
 * gates, asks for the causal Conv1D to be measurable on its own).
 *   x [B][T][C_ch], conv_w, conv_state (in/out) as above;
 *   qkv_out [B][T][C_ch] fp32: normalised and scaled q, normalised k, and v,
 *   all after conv + SiLU.  Updates conv_state to the last W-1 rows of
 *   concat(conv_state, x). */
GDN_API int gdn_conv1d(const gdn_dims *dims, int64_t T, const void *x, const void *conv_w,
               void *conv_state, float *qkv_out, void *stream);

/* The whole layer over 1 <= T <= 2^24 tokens per sequence, processed in
 * chunks of `chunk` in {16, 32, 64, 128} tokens (the last chunk may be
 * partial): the separately tuned GDN prefill behind the one semantic
 * interface ("Add a performance-parity Qwen3.8-27B Q4 and Q8 text backend on
 * Metal", section Scope), equal to token-by-token decode across chunk sizes
 * ("Implement the Qwen3.8 Flash Next Rust and Metal text core", section
 * Verification).
 * conv_state and rec_state carry the sequence in and out, so calls can be
 * chained: splitting a sequence at a multiple of `chunk` gives bit-identical
 * outputs and states.  `ws` is device workspace of at least
 * gdn_prefill_workspace_bytes(dims, T, chunk) bytes; its contents on entry
 * are ignored. */
GDN_API int gdn_prefill_chunked(const gdn_dims *dims, int64_t T, int32_t chunk, const void *x,
                        const void *z, const float *g, const float *beta,
                        const void *conv_w, void *conv_state, float *rec_state, void *y,
                        void *ws, size_t ws_bytes, void *stream);

/* The same function as gdn_prefill_chunked at T = 1, tuned for one token per
 * sequence: every recurrent state is streamed from HBM once and written back
 * once ("Add a performance-parity Qwen3.8-27B Q4 and Q8 text backend on
 * Metal", section Scope: separately tuned single-step decode behind the same
 * semantic interface as prefill).  Shapes as above with T = 1.  `ws`: at
 * least gdn_decode_workspace_bytes(dims) bytes (contents ignored). */
GDN_API int gdn_decode_step(const gdn_dims *dims, const void *x, const void *z, const float *g,
                    const float *beta, const void *conv_w, void *conv_state,
                    float *rec_state, void *y, void *ws, size_t ws_bytes, void *stream);

/* Slot-indexed decode of T = 1..4 tokens per sequence, with the state after
 * each token kept in a slot of its own, d = 128 only (sources: "Add Qwen3.8
 * MTP and multimodal inference on Metal without regressing text", section
 * Correctness gates: MTP candidate verification, cache updates and
 * rollback; the model card "Qwen3.8-27B FP8 + native MTP + multimodal Core
 * AI", section What is fused: a three-token target prefill; "Implement the
 * Qwen3.8 Flash Next Rust and Metal text core", implementation comment:
 * resident-state swaps).  Two launches, like gdn_decode_step: the conv step
 * for all T tokens, then one pass over the states that keeps them in
 * registers across the T tokens.  dims->B rows (sequences);
 *   x [B][T][C_ch], z [B][T][H_v][d_v], g, beta [B][T][H_v], y [B][T][H_v][d_v]
 *   as for prefill; conv_w as above;
 *   conv_pool [n_slots][W-1][C_ch] in_dtype and rec_pool
 *   [n_slots][H_v][d_v][d_k] fp32: a pool of conv histories and recurrent
 *   states, addressed by slot;
 *   in_slots [B] int32, device memory: the slot each sequence starts from;
 *   out_slots [B][T] int32, device memory, or NULL: the slot that receives
 *   the state (history and recurrent state) after token t of sequence b;
 *   NULL means the in slot after the last token and nothing before it.
 * The step equals T single-token decode steps; an MTP verifier passes
 * distinct out slots per token and afterwards keeps the slot of the last
 * accepted token (rollback without any copy).  A sequence whose in slot lies
 * outside [0, n_slots) is a padding row: its y rows are written as zero and
 * nothing else is touched; out slots outside that range are not stored.
 * Slot values live on the device and are not validated on the host.  One
 * sequence may use its in slot as an out slot; different sequences must not
 * share any slot (they would race).  `ws`: at least
 * T * gdn_decode_workspace_bytes(dims) bytes (contents ignored).  Errors:
 * GDN_ERR_INVALID_ARG for T outside 1..4, n_slots < 1 or a null in_slots. */
GDN_API int gdn_decode_multi(const gdn_dims *dims, int32_t T, const void *x, const void *z,
                             const float *g, const float *beta, const void *conv_w,
                             void *conv_pool, float *rec_pool, int32_t n_slots,
                             const int32_t *in_slots, const int32_t *out_slots, void *y,
                             void *ws, size_t ws_bytes, void *stream);

/* Packed variable-length prefill ("Implement the Qwen3.8 Flash Next Rust and
 * Metal text core", section Implementation: prefill/small-batch
 * infrastructure).  dims->B sequences, packed back to back:
 *   cu_seqlens [B+1] int64, HOST memory: sequence n owns token rows
 *   cu_seqlens[n] .. cu_seqlens[n+1]-1 (cu_seqlens[0] = 0, non-decreasing;
 *   a sequence may be empty; each at most 2^24 tokens);
 *   x [T_total][C_ch], z [T_total][H_v][d_v], g, beta [T_total][H_v],
 *   y [T_total][H_v][d_v] with T_total = cu_seqlens[B];
 *   conv_pool, rec_pool: state pools as for gdn_decode_multi (16-byte
 *   aligned); slots [B] int32, HOST memory: the slot of each sequence, in
 *   [0, n_slots) and pairwise distinct (checked; GDN_ERR_INVALID_ARG).
 * Each sequence gets exactly what gdn_prefill_chunked gives it alone, and its
 * slot holds its states afterwards; other slots are not touched.  `ws`: at
 * least gdn_prefill_varlen_workspace_bytes(dims, cu_seqlens, chunk) bytes
 * (min(3, non-empty sequences) times the largest single-sequence prefill
 * workspace; contents ignored).  Up to three sequences run at once: on
 * `stream` and on up to two auxiliary streams that the library creates on
 * the current device at the first such call and keeps until the process
 * ends (default priority), forked from and joined back to `stream` by
 * events, so the call stays ordered on `stream` like any other.  Concurrent
 * calls from several threads serialize on those streams. */
GDN_API size_t gdn_prefill_varlen_workspace_bytes(const gdn_dims *dims,
                                                  const int64_t *cu_seqlens, int32_t chunk);
GDN_API int gdn_prefill_varlen(const gdn_dims *dims, const int64_t *cu_seqlens, int32_t chunk,
                               const void *x, const void *z, const float *g, const float *beta,
                               const void *conv_w, void *conv_pool, float *rec_pool,
                               int32_t n_slots, const int32_t *slots, void *y, void *ws,
                               size_t ws_bytes, void *stream);

/* The GDN input projections, with the decay and beta parametrisation fused
 * into their epilogue ("Implement the Qwen3.8 Flash Next Rust and Metal text
 * core", section Verification: primitive vectors for the GDN projection).
 * One bf16 GEMM on the MFMA with fp32 accumulation over M = B * T token rows:
 *   h     [B][T][hidden] bf16 (hidden a multiple of 64; dims->in_dtype must
 *         be GDN_BF16);
 *   w_in  [C_ch + H_v*d_v + 2*H_v][hidden] bf16, rows in this order: the C_ch
 *         conv inputs x ([q | k | v], head-major, as for the layer), the
 *         H_v*d_v gate inputs z, H_v rows b, H_v rows a;
 *   A_log, dt_bias [H_v] fp32 (per value head);
 * outputs, laid out as the layer calls take them:
 *   x [B][T][C_ch] bf16, z [B][T][H_v][d_v] bf16 (the products rounded to
 *   bf16), beta [B][T][H_v] = sigmoid(b), g [B][T][H_v] = -exp(A_log) *
 *   softplus(a + dt_bias) fp32 (so the decay exp(g) lies in (0, 1)).
 * The decay and beta parametrisation is not on the pages; this is the
 * Mamba2-style gate of Gated DeltaNet.  All buffers 16-byte aligned (h,
 * w_in) or aligned to their element size (the rest); outputs must not
 * overlap the inputs. */
GDN_API int gdn_in_proj(const gdn_dims *dims, int64_t T, int32_t hidden, const void *h,
                        const void *w_in, const float *A_log, const float *dt_bias, void *x,
                        void *z, float *g, float *beta, void *stream);

/* The full-attention layer of the hybrid schedule (3 GDN : 1 attention):
 * Qwen RoPE, a bf16 KV cache and causal grouped-query attention ("Implement
 * the Qwen3.8 Flash Next Rust and Metal text core", section Implementation:
 * Qwen RoPE and an exact dense 24Q/2KV causal attention; its implementation
 * comment: BF16 KV storage; "Add a performance-parity Qwen3.8-27B Q4 and Q8
 * text backend on Metal", section Measurements and gates: full attention and
 * the hybrid block measured in isolation). */
typedef struct gdn_attn_dims {
  int32_t abi;        /* GDN_ABI_VERSION                                   */
  int32_t B;          /* sequences                                          */
  int32_t H_q, H_kv;  /* query heads, key/value heads (H_q % H_kv == 0)      */
  int32_t d_h;        /* head dimension: 128 or 256                         */
  int32_t rot_dim;    /* rotary width r (a multiple of 16, <= d_h)          */
  int32_t in_dtype;   /* q, k, v and the cache: GDN_BF16                    */
  int32_t out_dtype;  /* o: GDN_F32 or GDN_BF16                             */
  float rope_base;    /* RoPE base (> 1)                                    */
  float scale;        /* score scale, usually 1/sqrt(d_h)                   */
} gdn_attn_dims;

/* Attention over T new tokens per sequence at positions pos0 .. pos0+T-1,
 * with the cache's positions 0 .. pos0-1 as earlier context (pos0 = 0: a
 * fresh prefill; T = 1: one decode step at position pos0).
 *   q [B][T][H_q][d_h], k, v [B][T][H_kv][d_h] bf16 (before RoPE);
 *   k_cache, v_cache [B][T_max][H_kv][d_h] bf16, in/out: positions
 *   pos0 .. pos0+T-1 receive the rotated keys and the values;
 *   o [B][T][H_q][d_h] out_dtype.
 * RoPE (a reading of "Qwen RoPE"): the pairs (i, i + r/2), i < r/2, of the
 * first r dimensions turn by pos * rope_base^(-2i/r).  Query head h reads
 * KV head h / (H_q / H_kv); o = softmax(scale q k^T over the keys at
 * positions <= the query's) v, the softmax in fp32, the products on bf16
 * MFMA with fp32 accumulation.  pos0 + T <= T_max <= 2^24, and
 * B T (H_q + H_kv) d_h / 2 and 4 B H_q T + 512 B H_kv each below 2^31 (else GDN_ERR_INVALID_ARG; a single sequence at d_h = 256 with
 * 24 + 2 heads takes T up to 2^19 tokens).  `ws`: at least
 * gdn_attn_workspace_bytes(dims, T, pos0) bytes (contents ignored).  All
 * buffers 16-byte aligned (o: its element size); outputs, caches and
 * workspace must not overlap each other or the inputs. */
GDN_API size_t gdn_attn_workspace_bytes(const gdn_attn_dims *dims, int64_t T, int64_t pos0);
GDN_API int gdn_attn_prefill(const gdn_attn_dims *dims, int64_t T, int64_t pos0, const void *q,
                             const void *k, const void *v, void *k_cache, void *v_cache,
                             int64_t T_max, void *o, void *ws, size_t ws_bytes, void *stream);

/* Zero-centred grouped RMS norm before the sigmoid output gate ("Implement
 * the Qwen3.8 Flash Next Rust and Metal text core", section Implementation:
 * zero-centred norms; its implementation comment: zero-centred grouped RMS
 * and the sigmoid output gate), over the ungated readout of a layer call
 * (made with z = NULL and out_dtype GDN_F32).  For each of the rows * H_v
 * groups (one value head of one token, d_v values):
 *   y = o / sqrt(mean(o^2) + norm_eps) * (1 + norm_w) * sigmoid(z)
 *   o [rows][H_v][d_v] fp32; z [rows][H_v][d_v] in_dtype, or NULL (no gate);
 *   norm_w [d_v] fp32, the zero-centred weight shared by the heads, or NULL
 *   (all zero); y [rows][H_v][d_v] out_dtype; norm_eps >= 0.
 * o, z, norm_w and y 16-byte aligned; y must not overlap the inputs.
 * rows = B * T of the layer call (0: nothing to do). */
GDN_API int gdn_gated_rmsnorm(const gdn_dims *dims, int64_t rows, const float *o, const void *z,
                              const float *norm_w, float norm_eps, void *y, void *stream);

/* gdn_decode_step without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments (minus ws and ws_bytes) and the same results, bit for bit, as
 * gdn_decode_step; it runs the same kernels with the decode workspace placed
 * in a fixed 16 MiB device array that the library holds on each GPU it runs
 * on until the process ends.  Calls whose gdn_decode_workspace_bytes(dims)
 * exceeds 16 MiB (B above 409 at C_ch = 10240) are rejected with
 * GDN_ERR_TOO_LARGE before anything is enqueued.  The first call on a GPU
 * looks the array's device address up (no allocation, no stream work).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other threads) race and give wrong results;
 * calls in one stream order are safe.  Nothing in the array needs to start
 * at zero: each call writes what it reads. */
GDN_API int gdn_decode_step_noalloc(const gdn_dims *dims, const void *x, const void *z,
                                    const float *g, const float *beta, const void *conv_w,
                                    void *conv_state, float *rec_state, void *y, void *stream);

/* Measurement variants ("Add a performance-parity Qwen3.8-27B Q4 and Q8 text
 * backend on Metal", section Measurements and gates, asks for the conv, the
 * prefill, the decode and the recurrent-state update to be measured in
 * isolation).  Same arguments and effects as the plain calls, plus
 * `kernel_ms`, which receives the duration of each kernel of the call, taken
 * from HIP events recorded at the kernel's own start and end (an extended
 * launch, so the launch latency between kernels is not counted):
 *   prefill: [0] conv + L2 norm, [1] chunk-local prep (Gram, (I+A)^{-1}, P)
 *            and the conv history roll, [2] state pass + gate     (3 floats)
 *            (d = 128, chunk 64, more than 4096 chunk x key-head blocks:
 *            the q/k conv and norm run inside the prep launch, and [0]
 *            is 0)
 *   decode:  [0] conv step + L2 norm, [1] state stream + gate      (2 floats)
 * These variants create HIP events and wait for the last one before they
 * return. */
GDN_API int gdn_prefill_chunked_timed(const gdn_dims *dims, int64_t T, int32_t chunk,
                                      const void *x, const void *z, const float *g,
                                      const float *beta, const void *conv_w, void *conv_state,
                                      float *rec_state, void *y, void *ws, size_t ws_bytes,
                                      void *stream, float *kernel_ms);
GDN_API int gdn_decode_step_timed(const gdn_dims *dims, const void *x, const void *z,
                                  const float *g, const float *beta, const void *conv_w,
                                  void *conv_state, float *rec_state, void *y, void *ws,
                                  size_t ws_bytes, void *stream, float *kernel_ms);

/* Session checkpoint of every GDN conv and recurrent component with
 * versioned validation (issue #95, section Implementation).
 * Blob layout (little-endian): a 128-byte header
 *   [0,8)   magic "GDNSTATE"        [8,12)  format version (1)
 *   [12,16) header bytes (128)      [16,40) B, H_k, H_v, d_k, d_v, W (int32)
 *   [40,44) conv dtype              [44,48) recurrent dtype (GDN_F32)
 *   [48,56) conv bytes (uint64)     [56,64) recurrent bytes (uint64)
 *   [64,72) FNV-1a 64 of the payload  [72,80) FNV-1a 64 of bytes [0,72)
 *   [80,128) zero
 * followed by the conv_state bytes and the rec_state bytes, verbatim.
 * gdn_state_save writes the blob into host memory `blob` of blob_bytes ==
 * gdn_state_blob_bytes(dims) and returns once the copy has completed.
 * gdn_state_restore checks magic, version, header checksum, dims, dtypes,
 * sizes and payload checksum before it writes any device byte, then copies
 * the payload into conv_state and rec_state and waits for the copy. */
GDN_API int gdn_state_save(const gdn_dims *dims, const void *conv_state, const float *rec_state,
                   void *blob, size_t blob_bytes, void *stream);
GDN_API int gdn_state_restore(const gdn_dims *dims, const void *blob, size_t blob_bytes,
                      void *conv_state, float *rec_state, void *stream);

/* Host-only check of a blob against `dims` (the validation gdn_state_restore
 * runs first).  Touches no device. */
GDN_API int gdn_state_check(const gdn_dims *dims, const void *blob, size_t blob_bytes);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
