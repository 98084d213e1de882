/*
 * tq.h -- C ABI of libtq, compressed-domain KV-cache attention for MI355X
 * (gfx950): the TurboQuant / PolarQuant write path (quantize and append) and
 * read path (fused decode attention over the compressed bytes).
 *
 * Sources cited below by title and section:
 *   [P1] "turbo4 post-mortem": the turboquant_plus article on reviving the
 *        turbo4 KV-cache format, sections 1-10.
 *   [P2] "TurboQuant Triton deep dive": the article on the three tricks of
 *        the fused Triton decode kernels (nine-step path, tricks 1-3, how the
 *        kernels compose, write path).
 *   [P3] "PolarQuant-KV": the consumer-GPU KV-cache compression article,
 *        sections 1-6.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every call returns TQ_OK (0) or a negative tq_status.  Arguments are
 *   checked on the host before anything is enqueued; on an error nothing is
 *   enqueued and no device memory is touched.
 * - Device calls are asynchronous on the caller's HIP stream.  TQ_OK means
 *   "enqueued"; TQ_ERR_HIP reports a launch failure.  Faults surface at the
 *   caller's synchronization.
 * - The library allocates no device memory and keeps no mutable global
 *   state; it is reentrant across streams.  Every device buffer (caches,
 *   queries, outputs, workspace, the QJL matrix) is owned by the caller and
 *   passed as a raw device pointer.  Host structs are caller-owned PODs.
 * - Device pointers to caches and workspaces must be 16-byte aligned; fp32
 *   arrays 4-byte aligned.
 * - Cache layout: k_cache[B][Hkv][capacity][k_bytes_per_vector] (and the same
 *   for v_cache), so each (b, kv-head) stream is one contiguous byte run;
 *   capacity must be a multiple of 64.
 * - Grouped-query attention: query head g reads KV head g / (Hq / Hkv).
 * - Supported head dims: 128 and 256.  Supported format pairs
 *   (K, V): (PQ4, PQ4), (PQ3, PQ3), (PQ3, PQ4), (TQ3K, GQ2V), (TQ3K, GQ4V).
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tq_status {
    TQ_OK = 0,
    TQ_ERR_INVALID = -1,     /* null pointer, bad shape, misaligned buffer   */
    TQ_ERR_UNSUPPORTED = -2, /* head dim, bit width or format pair not built */
    TQ_ERR_WORKSPACE = -3,   /* workspace smaller than required              */
    TQ_ERR_RANGE = -4,       /* a size exceeds what the call can address     */
    TQ_ERR_HIP = -5          /* a HIP launch reported an error               */
} tq_status;

/* Cache formats.  Byte layouts (fp16 fields little-endian):
 *
 * TQ_FMT_PQ4  4-bit PolarQuant, the 68-byte turbo4 block of [P1] sections 5
 *             and 7: per 128 coordinates [fp16 norm][2 reserved bytes = 0]
 *             [qs: 64 B], code j in byte j/2, low nibble when j is even
 *             ([P1] section 5 prints (qs[j/2] >> ((j%2)*4)) & 0xF).
 *             d = 256 is two such blocks, each holding the full-vector norm.
 *             4.25 bits per value.
 * TQ_FMT_PQ3  turbo3, 3-bit codes in the byte-aligned "2+1" split of [P1]
 *             sections 2 and 4: per 32 coordinates [fp16 norm][qs: 8 B]
 *             [signs: 4 B] = 14 B; low bits (qs[j/4] >> ((j%4)*2)) & 3, high
 *             bit signs[j/8] bit j%8.  Rotation and norm span the whole
 *             vector; each 32-block repeats the vector norm.  3.5 bits/value.
 * TQ_FMT_TQ3K TurboQuant "prod" key ([P2] trick 2, [P1] sections 1-2): 2-bit
 *             MSE code plus a 1-bit QJL sign per coordinate:
 *             [fp16 norm][fp16 residual norm][qs: d/4 B, code j at bits
 *             2(j%4) of byte j/4][qjl: d/8 B, bit i at bit i%8 of byte i/8].
 *             52 B for d = 128.  Keys only.
 * TQ_FMT_GQ2V 2-bit asymmetric group quantization of values in groups of 32
 *             channels ([P2] trick 3 and write path, v*scale + zero):
 *             per group [fp16 scale][fp16 zero][q: 8 B packed like the PQ3
 *             low bits].  48 B for d = 128.  Values only.
 * TQ_FMT_GQ4V the same group quantization with 4-bit codes, for values where
 *             the 2-bit codes limit quality ([P2] write path: the value cache
 *             is group-quantized at 2 or 4 bits; [P2] limits: 4-bit values
 *             for quality-sensitive use): per 32-channel group [fp16 scale]
 *             [fp16 zero][q: 16 B, channel j in byte j/2, low nibble when j is
 *             even, the PQ4 nibble order]; scale = fp16(fp32(max - min)/15).
 *             80 B for d = 128.  Values only.
 */
typedef enum tq_format {
    TQ_FMT_PQ4 = 1,
    TQ_FMT_PQ3 = 2,
    TQ_FMT_TQ3K = 3,
    TQ_FMT_GQ2V = 4,
    TQ_FMT_GQ4V = 5
} tq_format;

/* Codebook constructions for the rotated-coordinate law N(0, 1/d)
 * ([P1] section 5; [P2] write path; [P3] section 2.2):
 *   TQ_CB_QUANTILE_MEAN  conditional mean of each of 2^bits equal-probability
 *                        intervals (the construction whose d = 128, 16-level
 *                        values [P1] section 5 prints);
 *   TQ_CB_LLOYD_MAX      fixed point of the Lloyd conditions (midpoint
 *                        boundaries, conditional-mean centroids).          */
typedef enum tq_codebook_kind {
    TQ_CB_QUANTILE_MEAN = 0,
    TQ_CB_LLOYD_MAX = 1
} tq_codebook_kind;

/* A codebook plus the rotation state of one tensor (keys or values).
 * Filled by tq_build_codebook; plain data, safe to copy.
 *   centroids[k]  fp32 centroid of code k (k < 2^bits), odd-symmetric
 *   bounds[k]     fp32 boundary between codes k and k+1: the fp32 rounding of
 *                 the float64 midpoint.  Code of y = number of bounds < y
 *                 (a value on a boundary takes the lower code).
 *   sign_bits     bit j set <=> rotation sign s_j = -1.  The rotation is
 *                 Pi = H_d diag(s) / sqrt(d), H_d Sylvester-ordered.
 * Formats without rotation or centroids (GQ2V) ignore the table.          */
typedef struct tq_codebook {
    int32_t head_dim;
    int32_t bits;
    int32_t kind;
    int32_t n_levels;
    float centroids[16];
    float bounds[16];
    uint32_t sign_bits[8];
    uint64_t rot_seed;
    uint64_t qjl_seed;
} tq_codebook;

/* Shape of one cache pair (K and V) and of the queries that read it. */
typedef struct tq_layout {
    int32_t batch;      /* B: sequences                                    */
    int32_t n_q_heads;  /* Hq: query heads, a multiple of n_kv_heads        */
    int32_t n_kv_heads; /* Hkv                                              */
    int32_t head_dim;   /* d: 128 or 256                                    */
    int32_t capacity;   /* tokens per (b, kv-head) stream, multiple of 64;
                           (capacity + 4096) * vector bytes < 2^31 (one
                           stream addressed with 32-bit offsets), and
                           batch * n_kv_heads * capacity < 2^31 (else
                           TQ_ERR_RANGE)                                  */
    int32_t k_format;   /* tq_format of keys                                */
    int32_t v_format;   /* tq_format of values                              */
    int32_t reserved;   /* must be 0                                        */
} tq_layout;

/* Library version string (static storage). */
const char* tq_version(void);

/* Static text for a tq_status. */
const char* tq_strerror(int status);

/* Build a codebook and the rotation state, on the host.
 *   head_dim  128 or 256 (64 is also accepted for host-side use)
 *   bits      2, 3 or 4; kind a tq_codebook_kind
 *   rot_seed  seed of the rotation signs: s_j = -1 iff bit 63 of output j of
 *             the splitmix64 stream (Steele, Lea, Flood 2014) seeded with
 *             rot_seed is set
 *   qjl_seed  seed of the QJL matrix S, which must not share the rotation's
 *             randomness ([P1] section 10: QJL failed with correlated
 *             rotations); recorded in the codebook
 *   out       filled on success
 *   qjl_S     nullable host buffer of head_dim*head_dim floats: S row-major,
 *             N(0, 1) entries, entries 2t, 2t+1 from Box-Muller on outputs
 *             2t, 2t+1 of the qjl_seed stream, each mapped to the uniform
 *             ((x >> 11) + 0.5) * 2^-53, computed in double, rounded to fp32.
 * Deterministic; no device work.  Errors: TQ_ERR_INVALID (null out),
 * TQ_ERR_UNSUPPORTED (head_dim, bits or kind).                            */
int tq_build_codebook(int head_dim, int bits, int kind, uint64_t rot_seed, uint64_t qjl_seed,
                      tq_codebook* out, float* qjl_S);

/* Bytes of one encoded vector of a format at a head dim (0 if unsupported). */
size_t tq_vector_bytes(int format, int head_dim);

/* Bytes the caller allocates for k_cache and v_cache of layout L. */
int tq_cache_bytes(const tq_layout* L, size_t* k_bytes, size_t* v_bytes);

/* Quantize and append: the write path ([P1] section 1, norm -> normalize ->
 * rotate -> nearest centroid; [P1] section 2, SET_ROWS; [P2] write path).
 * For each token t < T and KV head h, the fp16 vectors k_new[t][h][:] and
 * v_new[t][h][:] are encoded in the K and V formats of L and written to row
 * dst_row[t] = b*capacity + pos of stream (b, h).  Rotated formats: norm n
 * (fp32, stored as fp16 saturated at 65504), u = x/n (u = 0 when n = 0),
 * y = Pi u, code = number of fp32 bounds below fp32 y.  TQ3K additionally
 * stores gamma = |r| of the unrotated residual r = u - Pi^T c[code] and the
 * signs [(S r)_i >= 0] ([P1] section 2; [P2] trick 2).  GQ2V stores
 * zero = min, scale = fp16(fp32(max - min)/3) per 32-channel group and codes
 * clamp(rint(fp32(v - zero) * fp32(1/scale)), 0, 3), or 0 when scale is 0;
 * GQ4V the same with 15 in place of 3.
 *   cbk, cbv   host codebooks of the K and V formats
 *   S_dev      device fp32 d*d QJL matrix (TQ3K keys), else ignored
 *   k_new, v_new  device fp16 bits [T][Hkv][d]
 *   dst_row    device int32 [T]; rows outside [0, B*capacity) are skipped
 *   k_cache, v_cache  device caches of layout L
 * T = 0 enqueues nothing.  Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED,
 * TQ_ERR_RANGE (T * Hkv above 2^31 - 1), TQ_ERR_HIP.                      */
int tq_quantize_append(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv,
                       const float* S_dev, const uint16_t* k_new, const uint16_t* v_new,
                       const int32_t* dst_row, int T, void* k_cache, void* v_cache, hipStream_t stream);

/* Encode from given rotated coordinates: the quantize-and-pack half of the
 * write path alone, so that codes can be compared bit for bit with a
 * reference fed the same fp32 inputs.
 *   format  PQ4, PQ3 or TQ3K (for TQ3K the residual is Pi^T (y - c[code]))
 *   y       device fp32 [n][d], rotated coordinates of unit vectors
 *   norm16  device fp16 bits [n], stored as the vector norm
 *   S_dev   device QJL matrix for TQ3K, else ignored
 *   blocks  device output [n][tq_vector_bytes(format, d)], 16-byte aligned
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP.                  */
int tq_quantize_rotated(int format, const tq_codebook* cb, const float* S_dev, const float* y,
                        const uint16_t* norm16, int n, void* blocks, hipStream_t stream);

/* Rotate each query once and, for TQ3K keys, sketch it once ([P2] trick 1:
 * <q, Pi^T y> = <Pi q, y>, so the d x d work drops from once per key to once
 * per query; trick 2: q_sketch = S q reused for every key).
 *   q         device fp32 [B][Hq][d]
 *   q_rot     device fp32 [B][Hq][d] out: Pi q with the K codebook's signs
 *   q_sketch  device fp32 [B][Hq][d] out, required iff keys are TQ3K: S q
 *   S_dev     device QJL matrix, required iff keys are TQ3K
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP.                  */
int tq_rotate_sketch_query(const tq_layout* L, const tq_codebook* cbk, const float* S_dev,
                           const float* q, float* q_rot, float* q_sketch, hipStream_t stream);

/* Number of context splits and workspace bytes of a decode call.
 *   split_tokens  tokens per split, a multiple of 256, or 0 for the
 *                 library's choice (enough splits to fill the GPU).  Each
 *                 wavefront sums its share of a split in fp32, so the sums'
 *                 rounding grows with the split: on streams of tens of
 *                 millions of tokens a smaller split (such as 8192) keeps it
 *                 near 1e-4 of the output
 * Workspace layout (each region starts at a multiple of 256 bytes):
 *   float2 ml[B][Hq][splits]  (m, l) of every split record
 *   float  acc[B][Hq][splits][d]
 *   uint32 arrivals[B][Hkv]   per-stream arrival counters of the one-launch
 *                             decode (tq_decode_step with an output), which
 *                             merges the records in the launch that writes
 *                             them ([P2] trick 3: the split states are
 *                             combined once at the end); they must be zero
 *                             when such a decode starts, and every such
 *                             decode leaves them zero.
 *                             tq_decode_workspace_init clears them once
 *                             after allocation (a zero-filled allocation
 *                             does too).
 * Returns 0 on invalid input.                                             */
int tq_decode_splits(const tq_layout* L, int split_tokens);
size_t tq_decode_workspace_bytes(const tq_layout* L, int split_tokens);

/* Clear the arrival counters of a workspace (a fill kernel on `stream`, so
 * the call may be captured in a graph).  Needed once after allocation before
 * tq_decode_step with an output; the records need no initialization.  Errors: TQ_ERR_INVALID (layout, split length, null or
 * misaligned ws), TQ_ERR_WORKSPACE (ws_bytes too small), TQ_ERR_HIP.     */
int tq_decode_workspace_init(const tq_layout* L, int split_tokens, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* Fused decode attention over the compressed caches, one query token per
 * sequence: for query head g of sequence b, with h = g / (Hq/Hkv) and
 * N = seq_lens[b],
 *     s_i = <q, k_hat_i> / sqrt(d),  o = sum_i softmax(s)_i v_hat_i,  i < N,
 * where k_hat, v_hat are the dequantized cache rows.  Only compressed bytes
 * are read: scores accumulate q_rot[j] * c[code_j] per block and are scaled
 * by the block norm ([P2] trick 1), TQ3K adds
 * sqrt(pi/2)/d * gamma * <q_sketch, 2b - 1> ([P2] trick 2), an online
 * softmax (m, l, acc) runs over the keys and values are dequantized in
 * registers ([P2] trick 3); rotated values are accumulated in the rotated
 * basis and rotated back once per output ([P1] section 9, rotated V).
 *   q_rot, q_sketch  from tq_rotate_sketch_query (q_sketch only for TQ3K)
 *   seq_lens    device int32 [B], each in [0, capacity]; N = 0 gives o = 0
 *   out         device fp32 [B][Hq][d]
 *   scores      nullable device fp32 [B][Hq][capacity]: if given, s_i is
 *               written for i < N (the score-only path of [P2] tricks 1-2)
 *   split_tokens  as for tq_decode_splits
 *   ws, ws_bytes  device workspace of at least tq_decode_workspace_bytes
 * Equivalent to tq_decode_partial followed by tq_decode_combine (two
 * launches; tq_decode_step with an output merges in one launch instead).
 * Errors: TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
int tq_decode_attention(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv,
                        const float* q_rot, const float* q_sketch, const void* k_cache,
                        const void* v_cache, const int32_t* seq_lens, float* out, float* scores,
                        int split_tokens, void* ws, size_t ws_bytes, hipStream_t stream);

/* First half of tq_decode_attention: one online-softmax record per
 * (b, query head, split) in the workspace ([P2] trick 3: m_i, l_i, acc).
 * Records: float2 ml[B][Hq][splits] = (m, l) with m the running maximum of
 * s_i * log2(e) (-inf for an empty split) and l = sum 2^(s_i log2 e - m);
 * then float acc[B][Hq][splits][d] = sum 2^(s_i log2 e - m) v_hat_i, kept
 * in the rotated basis (Pi v_hat) for PQ4/PQ3 values.  These records are
 * what a context-sharded multi-device decode would exchange.               */
int tq_decode_partial(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv,
                      const float* q_rot, const float* q_sketch, const void* k_cache,
                      const void* v_cache, const int32_t* seq_lens, float* scores,
                      int split_tokens, void* ws, size_t ws_bytes, hipStream_t stream);

/* tq_decode_partial with HIP events attached to the kernel's own dispatch
 * (hipExtLaunchKernel): start and stop, created by the caller, are recorded
 * when the kernel begins and ends, so hipEventElapsedTime(start, stop) is the
 * kernel's duration without the queue and event-packet gaps around it.  For
 * profiling callers.  Errors: those of tq_decode_partial, and TQ_ERR_INVALID
 * for a null event.                                                        */
int tq_decode_partial_timed(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv,
                            const float* q_rot, const float* q_sketch, const void* k_cache,
                            const void* v_cache, const int32_t* seq_lens, float* scores,
                            int split_tokens, void* ws, size_t ws_bytes, hipStream_t stream,
                            hipEvent_t start, hipEvent_t stop);

/* The partial from the unrotated query: the query rotation of
 * tq_rotate_sketch_query ([P2] trick 1: <q, Pi^T y> = <Pi q, y>, rotate once
 * per query) followed by tq_decode_partial, in one call.  Where the kernel
 * can (PQ4 keys and values at d 128, four query heads per KV head, one
 * centroid table for K and V) it rotates the query in its own prologue, with
 * the same arithmetic, so the records equal those of the two calls bit for
 * bit and one launch is saved; otherwise the rotation runs as its own launch
 * into q_rot_scratch first.
 *   q              device fp32 [B][Hq][d], unrotated, 16-byte aligned
 *   q_rot_scratch  device fp32 [B][Hq][d], caller-owned, 16-byte aligned;
 *                  holds the rotated query after the call when the rotation
 *                  ran as its own launch, untouched otherwise
 *   start, stop    optional events attached to the partial kernel's own
 *                  dispatch (both or neither), as tq_decode_partial_timed
 * Other arguments as tq_decode_partial.  Errors: those of tq_decode_partial;
 * TQ_ERR_UNSUPPORTED for TQ3K keys (their scores need the query sketch: use
 * tq_rotate_sketch_query and tq_decode_partial); TQ_ERR_INVALID for a null
 * or misaligned q or scratch, or one event without the other.             */
int tq_decode_partial_from_query(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv,
                                 const float* q, float* q_rot_scratch, const void* k_cache,
                                 const void* v_cache, const int32_t* seq_lens, float* scores,
                                 int split_tokens, void* ws, size_t ws_bytes, hipStream_t stream,
                                 hipEvent_t start, hipEvent_t stop);

/* One decode step: append one new token per (sequence, KV head), then the
 * partial from the unrotated query, as tq_ring_flush of a one-slot ring (the
 * write path of [P2]: quantize on the way in, [P1] section 5 format)
 * followed by tq_decode_partial_from_query, and with `out` the merge of
 * tq_decode_combine.  Where the kernel rotates the query itself (the layouts
 * named there) it also encodes and writes the new rows, with the write
 * kernel's arithmetic, so the cache bytes and the records equal those of the
 * separate calls bit for bit, in one launch.  With `out`, the PQ4 kernels at
 * d 128 (four query heads per KV head, or eight with one centroid table)
 * merge each (b, kv-head) stream's split records in the workgroup that
 * finishes the stream last, with the combine's arithmetic (the output equals
 * the combine's bit for bit at four heads per KV head), so the whole step is
 * one launch; other layouts run the combine after the partial.  One launch
 * saves the second launch but adds a tail of three memory round trips after
 * a stream's last workgroup (record stores, arrival, record loads); at
 * batch 8, 32/8 heads, 65,536 tokens the two launches of the separate calls
 * measured 1.7 us less per step.  Calls sharing a workspace must not overlap.
 *   k_new, v_new  device fp16 [B][Hkv][d], 16-byte aligned
 *   new_pos       device int32 [B]: position of sequence b's new token;
 *                 < 0, or >= capacity, skips the sequence.  seq_lens must
 *                 count the new token when it is to be attended.
 *   out           nullable device fp32 [B][Hq][d]: the attention output;
 *                 then the workspace's arrival counters must be zero
 *                 (tq_decode_workspace_init).  Null: records only.
 * Other arguments as tq_decode_partial_from_query (k_cache and v_cache are
 * written); the events bracket the partial kernel (which holds the merge in
 * the one-launch case).  Errors: those of tq_decode_partial_from_query,
 * TQ_ERR_INVALID for null or misaligned new rows, positions or output.    */
int tq_decode_step(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const void* k_new,
                   const void* v_new, const int32_t* new_pos, const float* q, float* q_rot_scratch,
                   void* k_cache, void* v_cache, const int32_t* seq_lens, float* out, float* scores,
                   int split_tokens, void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t start,
                   hipEvent_t stop);

/* Sparse V.  [P1] "turbo4 post-mortem", section 9 (current state) lists a
 * sparse-V mode as active alongside the 4-bit format; the page gives no rule
 * or threshold.  Reading taken here: the value of a token is skipped when its
 * weight against the running maximum is negligible.  Exactly: with m the
 * running reference maximum of the wavefront that processes token t (never
 * above the split's true maximum), the token adds its weight e^(s_t - m) to
 * the denominator always, and its value times that weight to the accumulator
 * only when e^(s_t - m) >= v_threshold; a tile of tokens none of whose values
 * survive skips its value decode and products.  Since m is at most the row
 * maximum M, a skipped token has softmax weight p_t < v_threshold, so every
 * output coordinate j moves by at most sum_{t: p_t < v_threshold} p_t |v_tj|;
 * tokens with p_t >= v_threshold are always kept.  Which tokens below the
 * threshold are skipped depends on the order the kernel visits them.
 * Arguments, layout and errors as tq_decode_partial; v_threshold in [0, 1]
 * (else TQ_ERR_INVALID, NaN included).  v_threshold = 0 gives the results of
 * tq_decode_partial bit for bit.  The records feed tq_decode_combine.     */
int tq_decode_partial_sparse_v(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv,
                               const float* q_rot, const float* q_sketch, const void* k_cache,
                               const void* v_cache, const int32_t* seq_lens, float* scores,
                               int split_tokens, float v_threshold, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* Second half: merge the split records (m = max m_p, l = sum l_p 2^(m_p-m),
 * acc = sum acc_p 2^(m_p - m)), normalize o = acc / l (o = 0 when l = 0) and
 * rotate back with the V codebook's signs for PQ4/PQ3 values.              */
int tq_decode_combine(const tq_layout* L, const tq_codebook* cbv, int split_tokens, const void* ws,
                      size_t ws_bytes, float* out, hipStream_t stream);

/* Decode attention that allocates nothing, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid allocation): tq_decode_attention (without scores) with its
 * workspace in a library-owned device array of TQ_STATIC_SCRATCH_BYTES bytes,
 * one copy per GPU, held until the process ends.  The call runs on the
 * current device; its first call on a device looks up that device's copy.
 * Every call on a GPU shares that GPU's array and leaves the last call's split
 * records in it, so calls that overlap on one GPU (other streams, other host
 * threads) race; nothing in the array needs to start at zero.  The caller
 * still owns and passes inputs and outputs, as for tq_decode_attention.
 * Errors: those of tq_decode_attention; TQ_ERR_WORKSPACE, before any device
 * work, when tq_decode_workspace_bytes(L, split_tokens) exceeds
 * TQ_STATIC_SCRATCH_BYTES; TQ_ERR_HIP if the array cannot be found.      */
#define TQ_STATIC_SCRATCH_BYTES (8u << 20)
int tq_decode_attention_static(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv,
                               const float* q_rot, const float* q_sketch, const void* k_cache,
                               const void* v_cache, const int32_t* seq_lens, float* out, int split_tokens,
                               hipStream_t stream);

/* ---- Capture ring and hybrid attention --------------------------------
 * [P2] "write path": the capture step keeps the newest tokens exact in a
 * ring buffer and quantizes the oldest batch into compressed blocks only
 * when the ring is full, so no per-token quantization runs on the decode
 * path; [P2] "limits" names the hybrid mode, which attends over the exact
 * recent tokens and the compressed history together.
 *
 * Ring: fp16 k_ring[B][Hkv][ring_cap][d] and v_ring alike, caller-owned
 * (tq_ring_bytes each), 16-byte aligned.  The token at absolute position pos
 * of sequence b lives in slot pos % ring_cap.  1 <= ring_cap <=
 * TQ_RING_CAP_MAX.  The caller keeps, per sequence, comp_len (tokens
 * 0 .. comp_len-1 are in the compressed cache) and ring_len (tokens
 * comp_len .. comp_len+ring_len-1 are in the ring).                        */
#define TQ_RING_CAP_MAX 256

/* Bytes of one ring tensor; 0 for an invalid layout or capacity.           */
size_t tq_ring_bytes(const tq_layout* L, int ring_cap);

/* Copy one new fp16 K and V row per (sequence, KV head), k_new/v_new
 * [B][Hkv][d], into ring slot pos[b] % ring_cap (pos: device int32 [B], the
 * token's absolute position; pos < 0 skips the sequence).  No
 * quantization.  Errors: TQ_ERR_INVALID (null or misaligned pointer, bad
 * ring_cap), TQ_ERR_HIP.                                                  */
int tq_ring_append(const tq_layout* L, int ring_cap, const uint16_t* k_new, const uint16_t* v_new,
                   const int32_t* pos, void* k_ring, void* v_ring, hipStream_t stream);

/* Flush: quantize ring tokens first[b] .. first[b]+count-1 of every
 * sequence (first: device int32 [B]; normally the oldest count tokens) and
 * write their blocks at those positions of the compressed caches, exactly
 * as tq_quantize_append would.  A sequence with first < 0, and positions
 * at or past capacity, are skipped.  0 <= count <= ring_cap; count = 0
 * enqueues nothing.  Errors: as tq_quantize_append, TQ_ERR_INVALID for a
 * bad ring_cap or count.                                                   */
int tq_ring_flush(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv, const float* S_dev,
                  int ring_cap, const void* k_ring, const void* v_ring, const int32_t* first, int count,
                  void* k_cache, void* v_cache, hipStream_t stream);

/* Workspace of tq_decode_attention_hybrid: the split records alone (equal
 * to tq_decode_workspace_bytes; the ring needs no record of its own).      */
size_t tq_decode_hybrid_workspace_bytes(const tq_layout* L, int split_tokens);

/* Hybrid decode: softmax attention of every query over the compressed
 * tokens 0 .. comp_lens[b]-1 and the exact ring tokens comp_lens[b] ..
 * comp_lens[b]+ring_lens[b]-1 together (comp_lens, ring_lens: device int32
 * [B]; ring_lens is clamped to [0, ring_cap]).  The compressed part runs
 * the split-K decode; the ring part scores exact fp16 keys against the
 * unrotated query (Pi^T q_rot) and sums exact fp16 values inside the
 * combine, which merges them with the split records (two launches).  Both
 * empty: out = 0.  ws: tq_decode_hybrid_workspace_bytes.  Errors: as
 * tq_decode_attention, TQ_ERR_INVALID for a bad ring argument.              */
int tq_decode_attention_hybrid(const tq_layout* L, const tq_codebook* cbk, const tq_codebook* cbv,
                               const float* q_rot, const float* q_sketch, const void* k_cache,
                               const void* v_cache, const int32_t* comp_lens, int ring_cap,
                               const void* k_ring, const void* v_ring, const int32_t* ring_lens,
                               float* out, int split_tokens, void* ws, size_t ws_bytes,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
