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
 *    keeps no state between calls and is safe to call from several threads.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Compute calls
 *    only enqueue work and never synchronise; save/restore return after the
 *    copy has completed.
 *  - conv_state and rec_state are updated in place.  Outputs and workspace
 *    must not overlap any input or state buffer.
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

/* Element types. */
#define GDN_F32 0
#define GDN_BF16 1

/* Geometry and numeric options, passed by pointer to every call.
 * Built geometries: d_k = d_v in {16, 128}, W = 4, H_v a multiple of H_k,
 * in_dtype and out_dtype in {GDN_F32, GDN_BF16}, l2_eps >= 0. */
typedef struct gdn_dims {
  int32_t abi;       /* must be GDN_ABI_VERSION                     */
  int32_t B;         /* sequences                                    */
  int32_t H_k, H_v;  /* key heads, value heads                       */
  int32_t d_k, d_v;  /* head dimensions                              */
  int32_t W;         /* conv taps                                    */
  int32_t in_dtype;  /* x, z, conv_w, conv_state                     */
  int32_t out_dtype; /* y                                            */
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

/* The whole layer over T >= 1 tokens per sequence, processed in chunks of
 * `chunk` in {16, 32, 64, 128} tokens (the last chunk may be partial).
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
 * once.  Shapes as above with T = 1.  `ws`: at least
 * gdn_decode_workspace_bytes(dims) bytes. */
GDN_API int gdn_decode_step(const gdn_dims *dims, const void *x, const void *z, const float *g,
                    const float *beta, const void *conv_w, void *conv_state,
                    float *rec_state, void *y, void *ws, size_t ws_bytes, void *stream);

/* Measurement variants ("Add a performance-parity Qwen3.8-27B Q4 and Q8 text
 * backend on Metal", section Measurements and gates, asks for the conv, the
 * prefill, the decode and the recurrent-state update to be measured in
 * isolation).  Same arguments and effects as the plain calls, plus
 * `kernel_ms`, which receives the duration of each kernel launch of the call,
 * taken from HIP events that the library records on `stream` between its
 * launches:
 *   prefill: [0] conv + L2 norm, [1] chunk-local prep (Gram, (I+A)^{-1}, P)
 *            and the conv history roll, [2] state pass + gate     (3 floats)
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
