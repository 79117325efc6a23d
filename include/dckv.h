/*
 * dckv.h - C ABI of the DCKV prompt-KV-cache codec for AMD Instinct MI355X
 * (gfx950).
 *
 * The codec follows the DCKV digest page ("DCKV: Learned Transform Coding of
 * the Prompt KV Cache in Hybrid Language Models", trove.briskstack.com),
 * section "How it works":
 *   - each coded token's pre-RoPE keys and values of the full-attention
 *     layers form one row of D = n_layers * 2 * n_kv_heads * head_dim bf16
 *     values (6,144 for the paper's model); the first keep_head and the last
 *     keep_tail positions stay in bf16 (first paragraph);
 *   - one shared basis projects a row to n_coef = 2,048 coefficients; the
 *     synthesis side adds one hidden layer of 256 GELU units (Transform);
 *   - per-component quantisation steps; components whose Laplace scale is
 *     below 0.05 steps are dropped (Transform);
 *   - the codes go through a rANS coder with discretised-Laplace symbol
 *     models; a code outside [-127, 127] is stored as a 64-bit record
 *     instead (Coding);
 *   - even positions take their code means from the token's input embedding,
 *     odd positions also from both decoded neighbours, so decoding takes two
 *     parallel passes at any length; token ids are side information, not
 *     stored (Conditional entropy models);
 *   - RoPE is reapplied to the keys after decoding (first paragraph).
 *
 * Conventions
 *   - bf16 values are passed as their uint16 bit patterns.
 *   - Pointers are HIP device pointers unless marked (host).
 *   - hip_stream is a hipStream_t passed as void* (NULL = the null stream).
 *   - Every function returns DCKV_OK or a negative dckv_status.  Argument and
 *     size errors are returned synchronously and nothing is enqueued.  Errors
 *     that only the device can see are written to the call's device status
 *     word.  dckv_last_error() gives a message for the last failing call on
 *     the calling thread.
 *   - The library never allocates device memory on the encode/decode path:
 *     the caller passes a workspace of the size dckv_bytes() reports.
 *   - Only the shapes of the paper's codec are supported by the GPU kernels:
 *     n_layers = 6, n_kv_heads = 2, head_dim = 256 (D = 6144), n_coef = 2048,
 *     n_hidden = 256, emb_dim = 2048.  keep_head, keep_tail and rope_theta
 *     are free, vocab is below 2^19.  A request holds at most 2^18 positions.
 *   - The encode and decode calls issue no memset and no host
 *     synchronisation, so they can be captured in a HIP graph.
 *
 * Entry points, in the order below: plan (tables, creation, inspection,
 * mean table); sizing; encode; decode (rows, or the per-layer head
 * matrices); inverse RoPE of a post-RoPE cache; a paged attention cache on
 * either side; batches; the lossless stage alone; workspace views and kernel
 * timing; the closed-form fit of the conditional models; the training rate and
 * its gradients.
 */
#ifndef DCKV_H
#define DCKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dckv_plan_s dckv_plan_t; /* opaque; immutable after dckv_plan() */

typedef enum {
  DCKV_OK = 0,
  DCKV_EINVAL = -1,      /* bad argument, or a non-finite coefficient at encode */
  DCKV_ENOMEM = -2,      /* plan could not allocate its device tables */
  DCKV_ECAPACITY = -3,   /* stream capacity or workspace too small */
  DCKV_ECORRUPT = -4,    /* malformed stream, or a rANS group failed its end-state check */
  DCKV_EPLAN = -5,       /* stream was written under another plan (CRC / C_a mismatch) */
  DCKV_EHIP = -6,        /* a HIP runtime call failed */
  DCKV_EUNSUPPORTED = -7 /* shape or size outside what the kernels support */
} dckv_status;

/* Codec parameters.  Matrices are bf16 row-major device arrays owned by the
 * caller; they must stay alive and unchanged while any plan made from them
 * exists (embedding and mean_head are read only by dckv_plan()).  The three
 * vectors are read on the host during dckv_plan(). */
typedef struct {
  int32_t n_layers, n_kv_heads, head_dim;   /* 6, 2, 256 -> D = 6144 */
  int32_t n_coef, n_hidden, emb_dim, vocab; /* 2048, 256, 2048, 1 .. 2^19 - 1 */
  int32_t keep_head, keep_tail;             /* positions kept in bf16: 4, 128 */
  float rope_theta;                         /* RoPE base, e.g. 1e7 */
  const uint16_t *analysis;   /* A  [n_coef][D]          y = A x          */
  const uint16_t *synthesis;  /* S  [D][n_coef]          xhat = S yhat_b + W2 h_b */
  const uint16_t *w1;         /* W1 [n_hidden][n_coef]   h = GELU(W1 yhat_b) */
  const uint16_t *w2;         /* W2 [D][n_hidden]        (w1 = w2 = NULL: the
                                 linear codec, xhat = S yhat_b; streams are the same) */
  const uint16_t *embedding;  /* E  [vocab][emb_dim]     the LM's input embedding */
  const uint16_t *mean_head;  /* H  [n_coef][emb_dim]    mean = H E[tok]  */
  const float *nbr_weight;    /* (host) a_c [n_coef]: odd mean += a_c (yhat_{j-1,c} + yhat_{j+1,c}) */
  const float *laplace_scale; /* (host) b_c [n_coef] > 0, Laplace scale of component c */
  const float *base_step;     /* (host) delta_c [n_coef] > 0, trained quantisation step */
} dckv_params;

/* ---------------------------------------------------------------------------
 * Plan: the rate setting.  (DCKV digest, "How it works", Transform and Coding;
 * "What it claims": one trained codec per rate.)
 *
 * step_c = fp32(step_scale * delta_c); s_c = b_c / step_c (float64); component
 * c is active iff s_c >= 0.05; active components are ranked by ascending c.
 * For each active component the integer table over the codes -127..127 is the
 * zero-mean discretised Laplace of scale s_c restricted to +-127 and
 * renormalised, with 15-bit precision: f_k = 1 + floor(p_k / sum(p) * (2^15 -
 * 255)), the remainder added to f_0, p_0 = 1 - exp(-0.5/s),
 * p_k = (exp(-(|k|-0.5)/s) - exp(-(|k|+0.5)/s)) / 2, sum in index order.
 * The plan CRC is CRC-32 (zlib polynomial) over step (fp32 LE), the active
 * flags (u8) and the active tables' f (u16 LE, rank order).
 * --------------------------------------------------------------------------*/

/* Host only, no device needed: the plan's tables into caller buffers.
 * step_out (host) [n_coef], active_out (host) [n_coef], freq_out (host)
 * [n_coef][255] (rows 0..C_a-1 filled in rank order; may be NULL),
 * *c_active and *crc (host).  Returns DCKV_EINVAL for n_coef < 1,
 * non-positive or non-finite vectors, or a non-positive step_scale. */
int dckv_plan_tables(const float *base_step, const float *laplace_scale, int32_t n_coef,
                     float step_scale, float *step_out, uint8_t *active_out,
                     uint16_t *freq_out, int32_t *c_active, uint32_t *crc);

/* Builds a plan on the current HIP device, synchronously: host tables, an
 * upload of about 1.6 MB, and the embedding-mean table (below): vocab * n_coef
 * * 4 bytes (256 MiB for a 32,768-token vocabulary), computed with one GEMM on
 * the null stream, or shared with a live plan that has the same one
 * (dckv_plan_memory).  *out receives the handle;
 * free with dckv_plan_free.  Returns DCKV_EUNSUPPORTED for shapes the kernels
 * do not support (vocab above 2^19 - 1 among them: the encoder addresses the
 * mean table with 32-bit byte offsets), DCKV_ENOMEM when an allocation fails. */
int dckv_plan(const dckv_params *p, float step_scale, dckv_plan_t **out);
int dckv_plan_free(dckv_plan_t *plan);

/* Device memory a plan holds (host outputs, any pointer may be NULL):
 * *table_bytes, its own block of steps and integer tables (about 1.6 MB);
 * *mean_table_bytes, the embedding-mean table it uses (vocab * n_coef * 4);
 * *mean_table_users, how many live plans share that table.  Plans made on the
 * same device from the same embedding and mean_head arrays, the same vocab
 * and the same set of active components (so, the same column order) share
 * one table: dckv_plan builds it for the first and the last dckv_plan_free
 * releases it. */
int dckv_plan_memory(const dckv_plan_t *plan, uint64_t *table_bytes, uint64_t *mean_table_bytes,
                     int32_t *mean_table_users);

/* Host copies of the plan's tables (any pointer may be NULL). */
int dckv_plan_info(const dckv_plan_t *plan, float *step_out, uint8_t *active_out,
                   uint16_t *freq_out, int32_t *c_active, uint32_t *crc);

/* The plan's embedding-mean table (DCKV digest, "How it works", Conditional
 * entropy models: the code means of a position come from its token's input
 * embedding).  The mean of every coefficient depends on the token id alone,
 * so the plan holds it for the whole vocabulary:
 *   table[v][i] = sum_k E[v][k] * H[col_component[i]][k]   (fp32, bf16 inputs)
 * for v < vocab, row stride n_coef floats, where the columns are the active
 * components in rank order, then the dropped ones in ascending order.
 * *table (device, owned by the plan, valid until dckv_plan_free), *rows (host)
 * = vocab, col_component (host) [n_coef]; any pointer may be NULL. */
int dckv_plan_mean_table(const dckv_plan_t *plan, const float **table, int64_t *rows,
                         int32_t *col_component);

/* Pure host.  For a request of T tokens: the largest stream an encode can
 * produce and the workspace bytes that
 * dckv_encode / dckv_decode / the entropy stages need.  T <= 2^18 positions:
 * the kernels address each [T][D] operand through 32-bit byte offsets, so
 * longer requests return DCKV_EUNSUPPORTED (here and in every call that
 * takes T).  The workspace holds max(4096, N * C_a / 16) escape records
 * (6.25 % of the coded positions); an encode that finds more sets
 * DCKV_ECAPACITY.  So the largest stream is the fixed part plus, per coded
 * position, one 16-bit word or (for at most that many) one 8-byte record,
 * plus a 32-bit flush per substream. */
int dckv_bytes(const dckv_plan_t *plan, int64_t T, uint64_t *max_stream_bytes,
               uint64_t *workspace_bytes);

/* ---------------------------------------------------------------------------
 * Encode (DCKV digest, "How it works": all bullets; stream layout below).
 *
 * rows      [T][D] bf16 pre-RoPE rows, column ((l*2 + kv)*n_kv_heads + h)*head_dim + d
 *           with kv = 0 for keys.
 * token_ids [T] int32, each in [0, vocab).
 * Coded row j is position t = j + keep_head, j = 0..N-1, N = max(T - keep_head -
 * keep_tail, 0).  y_j = A x_t; mu_j = H E[tok_t] for even j and
 * H E[tok_t] + a (yhat_{j-1} + yhat_{j+1}) for odd j (yhat_N = 0); the code is
 * q = rint(fp32(y - mu) / step) (float32, ties to even) for active components,
 * yhat = mu + q step; |q| > 127 is escaped.  Codes of each (256-token block,
 * 64 active components) group are coded by an interleaved 32-bit rANS
 * (16-bit renormalisation, L = 2^16).
 * stream       output, `capacity` bytes.
 * stream_bytes (device) u64: the stream's size, or 0 on a device-side error.
 * status       (device) int32: DCKV_OK, DCKV_EINVAL (non-finite residual),
 *              DCKV_ECAPACITY (stream larger than capacity, or more escapes
 *              than the workspace holds).
 * Asynchronous on hip_stream.  capacity must be at least the fixed part
 * (header, kept rows and group offsets) or DCKV_ECAPACITY is returned.
 * --------------------------------------------------------------------------*/
int dckv_encode(const dckv_plan_t *plan, const uint16_t *rows, const int32_t *token_ids,
                int64_t T, uint8_t *stream, uint64_t capacity, uint64_t *stream_bytes,
                int32_t *status, void *workspace, uint64_t workspace_bytes, void *hip_stream);

/* ---------------------------------------------------------------------------
 * dckv_encode_noalloc: dckv_encode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and errors as dckv_encode, minus
 * the workspace: the library keeps a 72 MiB static device array per GPU it
 * runs on (held until the process ends), which covers a request of up to
 * 8,192 positions under any plan; a longer request returns DCKV_ECAPACITY
 * and enqueues nothing.  The call allocates nothing and issues no memset (the
 * kernels initialise what they read).  Every call on one GPU shares that
 * GPU's array and it keeps the last call's contents: calls that overlap on
 * one GPU (other streams, other threads) race and must be serialised by the
 * caller.  The first call on a device looks up the array's address there.
 * --------------------------------------------------------------------------*/
int dckv_encode_noalloc(const dckv_plan_t *plan, const uint16_t *rows, const int32_t *token_ids,
                        int64_t T, uint8_t *stream, uint64_t capacity, uint64_t *stream_bytes,
                        int32_t *status, void *hip_stream);

/* ---------------------------------------------------------------------------
 * Decode: two checkerboard passes, synthesis with the GELU correction, RoPE.
 * (DCKV digest, "How it works": Transform, Conditional entropy models, first
 * paragraph for RoPE.)
 *
 * stream, stream_bytes (host u64): a stream from dckv_encode.
 * token_ids [T] int32: the same ids that were encoded (not stored).
 * rows_out  [T][D] bf16: every row with RoPE applied to the key columns
 *           (rotate-half, w_i = theta^(-i/(head_dim/2)), angle t*w_i).
 * status    (device) int32: DCKV_OK, DCKV_ECORRUPT, DCKV_EPLAN.  On error the
 *           contents of rows_out are unspecified.
 * Asynchronous on hip_stream.
 * --------------------------------------------------------------------------*/
int dckv_decode(const dckv_plan_t *plan, const uint8_t *stream, uint64_t stream_bytes,
                const int32_t *token_ids, int64_t T, uint16_t *rows_out, int32_t *status,
                void *workspace, uint64_t workspace_bytes, void *hip_stream);

/* ---------------------------------------------------------------------------
 * dckv_decode_heads: dckv_decode into the attention layers' cache layout
 * instead of rows.  kv_out (host array of 2 * n_layers device pointers):
 * kv_out[2 l + kv] (kv = 0 keys, 1 values) receives a bf16 [n_kv_heads][T]
 * [head_dim] matrix, the columns ((l 2 + kv) n_kv_heads + h) head_dim + d of
 * every decoded row (keys with RoPE reapplied).  Same values as dckv_decode;
 * each matrix 16-byte aligned, caller-owned.  (The cache-layout integration
 * next to the hot path: the decoded cache lands where the attention reads it.)
 * --------------------------------------------------------------------------*/
int dckv_decode_heads(const dckv_plan_t *plan, const uint8_t *stream, uint64_t stream_bytes,
                      const int32_t *token_ids, int64_t T, uint16_t *const *kv_out, int32_t *status,
                      void *workspace, uint64_t workspace_bytes, void *hip_stream);

/* ---------------------------------------------------------------------------
 * dckv_unrope: the inverse of the RoPE that dckv_decode reapplies, so that a
 * post-RoPE cache can be encoded (DCKV digest, "How it works", first
 * paragraph: keys are coded before RoPE).  rows_in [T][D] bf16 at positions
 * 0..T-1 -> rows_out [T][D]: on the key columns (x0, x1) = (p0 c + p1 s,
 * p1 c - p0 s) for the pair (d, d + head_dim/2) at angle t w_d, computed in
 * fp64 and rounded once to bf16; value columns copied.  rows_out may equal
 * rows_in.  4-byte aligned device arrays.  Asynchronous on hip_stream.
 * --------------------------------------------------------------------------*/
int dckv_unrope(const dckv_plan_t *plan, const uint16_t *rows_in, int64_t T, uint16_t *rows_out, void *hip_stream);

/* ---------------------------------------------------------------------------
 * dckv_encode_postrope: dckv_encode of a cache whose keys already carry RoPE
 * (the form an attention layer keeps them in).  DCKV digest, "How it works",
 * first paragraph: the codec works on keys without their rotary embedding.
 * rows [T][D] bf16 at positions 0..T-1, key heads rotated at angle t w_d.
 * The call first rotates the key heads back into a key copy in the workspace
 * (the arithmetic of dckv_unrope: fp64, no fused products, one rounding to
 * bf16), then encodes with its key k-tiles from that copy and its value
 * k-tiles from rows, so the stream equals dckv_encode's of
 * dckv_unrope(rows) byte for byte.  The caller's rows are not modified.
 * Other arguments and errors as dckv_encode; the workspace must hold
 * dckv_bytes_postrope() bytes (the encode's part of dckv_bytes() plus
 * T * n_layers * n_kv_heads * head_dim * 2 bytes for the key copy).
 * --------------------------------------------------------------------------*/
int dckv_bytes_postrope(const dckv_plan_t *plan, int64_t T, uint64_t *workspace_bytes);
int dckv_encode_postrope(const dckv_plan_t *plan, const uint16_t *rows, const int32_t *token_ids,
                         int64_t T, uint8_t *stream, uint64_t capacity, uint64_t *stream_bytes,
                         int32_t *status, void *workspace, uint64_t workspace_bytes, void *hip_stream);

/* ---------------------------------------------------------------------------
 * A paged attention cache on either side of the codec (DCKV digest, "How it
 * works", first paragraph: the codec takes the keys before RoPE and reapplies
 * it after decoding; abstract page: the cache is stored or moved to reuse it).
 * Serving engines keep the cache in fixed-size blocks: per layer l a key pool
 * kv[2 l] and a value pool kv[2 l + 1], each bf16
 * [n_blocks][block_size][n_kv_heads][head_dim] (16-byte aligned, device), and
 * one block table per request: position t of the request lives at row
 * block_table[t / block_size] * block_size + t % block_size of every pool.
 * Row t of the codec is then, per layer, the position's key heads followed by
 * its value heads (the dckv_params row order).  The struct is host memory; the
 * block table (int32, ceil(T / block_size) entries) is device memory.
 *
 * dckv_encode_paged: dckv_encode of the request held in the pools.  post_rope
 * != 0: the keys carry RoPE at their positions and are rotated back first with
 * dckv_unrope's arithmetic, so the stream equals dckv_encode_postrope's of the
 * gathered rows; post_rope = 0: the stream equals dckv_encode's of them.  The
 * rows are gathered into the workspace (one read of the request's blocks).
 * dckv_decode_paged: dckv_decode, then the decoded rows (keys post-RoPE) are
 * written into the request's rows of the pools; no other row is touched.
 * Both: the workspace must hold dckv_bytes_paged() bytes (dckv_bytes()'s
 * workspace plus T * 12,288 bytes of rows, plus 256).  The block table is
 * checked on the device before the pools are used: an entry outside
 * [0, n_blocks) makes the call's status DCKV_EINVAL (encode: and *stream_bytes
 * 0), and then nothing is read from (encode) or written to (decode) the pools.
 * Other arguments, errors and asynchrony as dckv_encode / dckv_decode.
 * --------------------------------------------------------------------------*/
typedef struct dckv_paged_kv {
  uint16_t *kv[12];             /* kv[2 l + kv]: layer l's key (kv = 0) or value (1) pool */
  const int32_t *block_table;   /* (device) physical block of each of the request's blocks */
  int32_t block_size;           /* positions per block, >= 1 */
  int64_t n_blocks;             /* blocks in each pool, >= 1 */
} dckv_paged_kv;

int dckv_bytes_paged(const dckv_plan_t *plan, int64_t T, uint64_t *workspace_bytes);
int dckv_encode_paged(const dckv_plan_t *plan, const dckv_paged_kv *cache, int32_t post_rope,
                      const int32_t *token_ids, int64_t T, uint8_t *stream, uint64_t capacity,
                      uint64_t *stream_bytes, int32_t *status, void *workspace, uint64_t workspace_bytes,
                      void *hip_stream);
int dckv_decode_paged(const dckv_plan_t *plan, const uint8_t *stream, uint64_t stream_bytes,
                      const int32_t *token_ids, int64_t T, const dckv_paged_kv *cache, int32_t *status,
                      void *workspace, uint64_t workspace_bytes, void *hip_stream);

/* ---------------------------------------------------------------------------
 * Batches of independent requests in one call (DCKV digest, "How it works":
 * every request is coded on its own; "Limits": the pages code one request at a
 * time, so a batch is our extension).
 *
 * Each dckv_req describes one request; the array itself is host memory.
 *   plan         the request's plan (its rate); every plan on the same device
 *   rows         encode: [T][D] bf16 pre-RoPE rows (device); unused by decode
 *   token_ids    [T] int32 (device)
 *   T            the request's length
 *   stream       encode: output buffer; decode: the request's stream (device)
 *   capacity     encode: bytes available at stream; decode: the stream's size
 *   stream_bytes encode: (device) u64 receiving the stream's size (0 on a
 *                device-side error); unused by decode
 *   rows_out     decode: [T][D] bf16 output (device); unused by encode
 *   status       (device) int32 per request, as for dckv_encode / dckv_decode
 * Every request is checked before anything is enqueued: an argument error in
 * any request returns its code (dckv_last_error names the request) and
 * enqueues nothing.  The requests share one workspace of dckv_bytes_batch()
 * bytes, the sum of their dckv_bytes() needs (each rounded up to 256 bytes):
 * each request gets its own slice, and every stage runs in one launch over up
 * to 16 requests (the transform GEMMs over all the requests' tiles, the stream
 * stages over all their groups), so a batch is one launch sequence.
 * Everything is enqueued on
 * hip_stream; the workspace is owned by the caller and must not be used by
 * other work on other streams meanwhile.  Each request's results equal those
 * of the single-request call.
 * --------------------------------------------------------------------------*/
typedef struct dckv_req {
  const dckv_plan_t *plan;
  const uint16_t *rows;
  const int32_t *token_ids;
  int64_t T;
  uint8_t *stream;
  uint64_t capacity;
  uint64_t *stream_bytes;
  uint16_t *rows_out;
  int32_t *status;
} dckv_req;

int dckv_bytes_batch(const dckv_req *reqs, int32_t n, uint64_t *workspace_bytes);
int dckv_encode_batch(const dckv_req *reqs, int32_t n, void *workspace, uint64_t workspace_bytes,
                      void *hip_stream);
int dckv_decode_batch(const dckv_req *reqs, int32_t n, void *workspace, uint64_t workspace_bytes,
                      void *hip_stream);

/* ---------------------------------------------------------------------------
 * The lossless stage alone (DCKV digest, "How it works", Coding).
 *
 * dckv_entropy_encode: writes the stream for given codes.
 *   sym        [N][C_a] u8, symbol q+127 per active component (rank order),
 *              255 at escaped positions;
 *   esc        [n_esc] records {u32 flat = j*C_a + rank, i32 q}, strictly
 *              ascending flat, exactly the positions where sym == 255;
 *   rows       [T][D] bf16, only the kept rows are read;
 *   stream, capacity, stream_bytes, status as for dckv_encode.
 * dckv_entropy_decode: parses and rANS-decodes a stream.
 *   sym_out    [N][C_a] u8 (255 at escaped positions);
 *   n_esc_out  (device) u32: number of escape records (they are in the stream).
 *   status     (device) as for dckv_decode.
 * --------------------------------------------------------------------------*/
int dckv_entropy_encode(const dckv_plan_t *plan, int64_t T, const uint8_t *sym,
                        const uint32_t *esc, uint32_t n_esc, const uint16_t *rows,
                        uint8_t *stream, uint64_t capacity, uint64_t *stream_bytes,
                        int32_t *status, void *workspace, uint64_t workspace_bytes,
                        void *hip_stream);
int dckv_entropy_decode(const dckv_plan_t *plan, const uint8_t *stream, uint64_t stream_bytes,
                        int64_t T, uint8_t *sym_out, uint32_t *n_esc_out, int32_t *status,
                        void *workspace, uint64_t workspace_bytes, void *hip_stream);

/* ---------------------------------------------------------------------------
 * Introspection of the workspace after a call (for tests and tools).
 * Valid until the workspace is reused.  which:
 *   DCKV_VIEW_SYMBOLS  u8 symbols of the last encode, or of the last decode with
 *                      a plan that drops components (a decode with every
 *                      component coded dequantises inside the rANS decoder
 *                      and leaves this view unwritten; dckv_entropy_decode
 *                      returns the symbols), group-tiled:
 *                      [G][N256/4][64][4], N256 = 256 * ceil(N/256);
 *                      symbol (j, rank r) at ((r/64)*(N256/4) + j/4)*256 + (r%64)*4 + j%4
 *   DCKV_VIEW_YHAT_B   bf16 [N][n_coef] decoded coefficients (row stride n_coef)
 *   DCKV_VIEW_H_B      bf16 [N][n_hidden] correction hidden units
 * --------------------------------------------------------------------------*/
enum { DCKV_VIEW_SYMBOLS = 0, DCKV_VIEW_YHAT_B = 1, DCKV_VIEW_H_B = 2 };
int dckv_workspace_view(const dckv_plan_t *plan, int64_t T, int32_t which, uint64_t *offset,
                        uint64_t *bytes, int64_t *row_stride);

/* ---------------------------------------------------------------------------
 * Kernel timing.  While enabled, every launch of the named kernels is
 * bracketed by HIP events on the call's stream; dckv_profile_read()
 * synchronises those events and returns the summed milliseconds and the
 * number of launches since the last reset.  Kernel names:
 * "analysis_gemm", "rans_encode", "rans_decode", "dequant", "w1_gemm",
 * "w1_gelu", "synthesis_gemm", "fixup", "scan", "pack", "parse".
 * dckv_profile_only() restricts the timing to one kernel name (NULL or ""
 * restores all), so that a timed run carries two events per launch of that
 * kernel and none elsewhere.
 * --------------------------------------------------------------------------*/
int dckv_profile_enable(int32_t on);
int dckv_profile_only(const char *kernel);
int dckv_profile_reset(void);
int dckv_profile_read(const char *kernel, double *total_ms, int64_t *launches);

/* ---------------------------------------------------------------------------
 * Closed-form fit of the conditional models to a trained codec (DCKV digest,
 * Evidence: fitting them in closed form recovers a saving close to joint
 * training).  The page names no estimator; these are the plainest closed
 * forms for the models of "How it works", Conditional entropy models:
 *   - calibration: n consecutive coded rows x_j [n][D] (bf16) of one prompt
 *     with their token ids; y_j = A x_j, e_j = E[tok_j];
 *   - mean head, ridge least squares over all rows:
 *       H^T = (E^T E + ridge * n * I)^-1 E^T Y   -> mean_head_out, fp32
 *     [n_coef][emb_dim] (may be NULL) and mean_head_bf16_out, its bf16
 *     rounding, the form a plan takes (may be NULL);
 *   - with m_j = bf16(H) e_j and, for odd j, s_j = y_{j-1} + y_{j+1}
 *     (y_n = 0): nbr_weight_out[c] = sum r s / sum s^2 over the odd rows,
 *     r = y - m (0 if sum s^2 = 0);
 *   - laplace_scale_out[c] = mean over all rows of |y - mu|, mu = m, plus
 *     a s on odd rows (the Laplace maximum-likelihood scale).
 * Outputs are device arrays.  Uses analysis and embedding of p (its other
 * pointers may be NULL).  The fit runs in fp32 on bf16 MFMA products
 * (E^T Y keeps 16 mantissa bits of Y) with a blocked Cholesky solve; a Gram
 * matrix plus ridge that is not positive definite, or a token id outside
 * [0, vocab), sets *status to DCKV_EINVAL.  The workspace (dckv_fit_bytes)
 * is about 28 KiB per calibration row plus 57 MiB.  2 <= n <= 2^18.
 * --------------------------------------------------------------------------*/
int dckv_fit_bytes(int64_t n, uint64_t *workspace_bytes);
int dckv_fit(const dckv_params *p, const uint16_t *rows, const int32_t *token_ids, int64_t n, float ridge,
             float *mean_head_out, uint16_t *mean_head_bf16_out, float *nbr_weight_out, float *laplace_scale_out,
             int32_t *status, void *workspace, uint64_t workspace_bytes, void *hip_stream);

/* ---------------------------------------------------------------------------
 * Training rate: the code length of additive-noise coefficients and its
 * gradients (DCKV digest page, "How it works", Training bullet: the rate is
 * computed with additive noise, the reconstruction from rounded values whose
 * gradient passes straight through).  The distortion term of the training
 * loss needs the language model and is not part of this call.
 *
 * For coded row j (position t = j + keep_head, 0 <= j < N) and component c,
 * with the plan's step D_c, its Laplace scale b_c (the params' laplace_scale)
 * and s = b_c / D_c:
 *   y = A x_t (fp32 accumulation of bf16 products); m = H E[tok_t];
 *   mu = m for even j, m + a (yhat_{j-1} + yhat_{j+1}) for odd j (yhat_N = 0);
 *   yhat = mu + rint(fp32(y - mu) / D) D, the codec's two-pass reconstruction;
 *   t = (y - mu) / D + noise[j][c];
 *   bits = -log2(F_s(t + 1/2) - F_s(t - 1/2)), F_s the zero-mean Laplace CDF.
 * Dropped components (the plan's drop rule) have bits 0, yhat = mu and zero
 * gradients.  R is the sum of bits over rows and active components; with the
 * straight-through rule (d yhat / d y = 1, d yhat / d mu = 0):
 *   bits_out    [N]     fp32  per-token sum of bits
 *   yhat_out    [N][C]  fp32  reconstruction (components in natural order)
 *   grad_y      [N][C]  fp32  dR/dy, including the even rows' share in their
 *                             odd neighbours' means
 *   grad_mean   [N][C]  fp32  dR/dm (for the mean head's gradient)
 *   grad_nbr    [C]     fp32  dR/da
 *   grad_scale  [C]     fp32  dR/db
 * rows [T][D] bf16 pre-RoPE (16-byte aligned) and token_ids [T] are those of
 * dckv_encode; noise [N][C] fp32 is the caller's uniform draw in steps,
 * normally in [-1/2, 1/2).  All outputs and the workspace are caller-owned
 * device memory (4-byte aligned, workspace 256-byte aligned, at least
 * dckv_rate_bytes); nothing is allocated.  Arguments are checked
 * synchronously (negative return, nothing enqueued); a non-finite y - mu or a
 * token id outside [0, vocab) sets *status to DCKV_EINVAL on the device.
 * The workspace is about 8.3 KiB per coded row (16.3 KiB up to 4,096 coded
 * rows, where the transform is split in two k ranges).  T <= 2^18.
 * --------------------------------------------------------------------------*/
int dckv_rate_bytes(const dckv_plan_t *plan, int64_t T, uint64_t *workspace_bytes);
int dckv_rate_forward(const dckv_plan_t *plan, const uint16_t *rows, const int32_t *token_ids, int64_t T,
                      const float *noise, float *bits_out, float *yhat_out, float *grad_y, float *grad_mean,
                      float *grad_nbr, float *grad_scale, int32_t *status, void *workspace,
                      uint64_t workspace_bytes, void *hip_stream);

/* Weight gradients through the codec's transforms (same passage): with
 * y_j = A x_j and m_j = H e_j (x_j the coded row at t = j + keep_head, e_j the
 * input embedding of its token),
 *   grad_analysis  [n_coef][D]     fp32  = sum_j grad_y[j] x_j^T
 *   grad_mean_head [n_coef][emb]   fp32  = sum_j grad_mean[j] e_j^T
 * over the N coded rows.  grad_y and grad_mean ([N][n_coef] fp32) are any
 * upstream gradients, e.g. dckv_rate_forward's, plus a distortion term's.
 * The products run on the bf16 MFMA with fp32 accumulation; the gradients
 * enter as two bf16 halves (16 mantissa bits), rows and embeddings are exact.
 * Caller-owned device memory throughout (rows, grad_y and grad_mean 16-byte,
 * the outputs 4-byte aligned, workspace 256-byte aligned and at least
 * dckv_rate_backward_bytes,
 * about 32 KiB per coded row); a token id outside [0, vocab) sets *status to
 * DCKV_EINVAL.  T <= 2^18. */
int dckv_rate_backward_bytes(const dckv_plan_t *plan, int64_t T, uint64_t *workspace_bytes);
int dckv_rate_backward(const dckv_plan_t *plan, const uint16_t *rows, const int32_t *token_ids, int64_t T,
                       const float *grad_y, const float *grad_mean, float *grad_analysis, float *grad_mean_head,
                       int32_t *status, void *workspace, uint64_t workspace_bytes, void *hip_stream);

const char *dckv_last_error(void);

/* Stream layout, version 1 (little endian, sections contiguous, no padding):
 *   0   "DCKV", u16 version = 1, u16 header_bytes = 64
 *   8   u32 T, keep_head, keep_tail, N, n_coef, C_a, n_groups, n_esc
 *   40  f32 step_scale, u32 plan_crc
 *   48  u64 total_bytes, u64 rans_bytes
 *   64  kept rows, bf16 pre-RoPE, in position order: (T - N) rows of D
 *   ..  u32 group_offset[n_groups + 1], byte offsets into the rANS section
 *   ..  n_esc records {u32 flat, i32 q}, ascending flat
 *   ..  rANS section: group id = b*G + g (b = 256-token block, g = 64-component
 *       group, G = ceil(C_a/64)), each a sequence of u16 words.
 * A group's lanes are active ranks 64g..64g+n-1; its encoder starts each lane
 * at x = 2^16, codes tokens last to first and lanes last to first, emits
 * x & 0xFFFF and shifts by 16 while x >= f * 2^17, then
 * x = (x / f) * 2^15 + x % f + cum; it ends by emitting, lanes last to first,
 * x >> 16 then x & 0xFFFF; the stored words are the emitted ones reversed.
 * Escaped positions are skipped. */

#ifdef __cplusplus
}
#endif
#endif /* DCKV_H */
