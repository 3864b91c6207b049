/*
 * csa2.h -- C ABI of the CSA2 attention layer for MI355X (gfx950).
 *
 * One attention layer of Compressed Sparse Attention 2 on one GPU: pair-pooled
 * FP4 compressed keys, a 32-head lightning indexer choosing 512 entries per
 * query, a 128-token FP8 window, and 64-head shared-latent attention with a
 * per-head sink.  Every step runs in the library's own HIP kernels.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never frees them and allocates no device memory.  Scratch memory comes
 *    from the caller's workspace (see csa2_workspace_size).
 *  - bf16 tensors are passed as uint16_t bit patterns.  Layouts are row-major
 *    in the bracketed order.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; no call synchronises.
 *  - Positions are absolute token positions.  `ratio` is the number of
 *    positions per compressed entry [zharf, CSA2 section: compression ratio
 *    one is a supported case; the decoder layers use it]:
 *      ratio 2: entry j pools the tokens at positions 2j and 2j+1 and is
 *               rotated at position 2j; a query at p sees j < floor((p+1)/2);
 *      ratio 1: entry j is the token at position j alone (the pooling softmax
 *               over one logit is 1, so no gate logits are read), rotated at
 *               j; a query at p sees j <= p.
 *    Any other ratio returns CSA2_ERR_UNSUPPORTED.
 *  - Caches (per request b, `entry_stride` entries apart):
 *      z_codes  [B][entry_stride][256]  E2M1 pairs, element 2i in the low nibble of byte i
 *      z_scales [B][entry_stride][16]   z_format 0: E8M0 bytes, one per 32 channels
 *                                       (2^(byte-127)); 272 bytes per entry
 *               [B][entry_stride][32]   z_format 1, the pages' format [zharf, "Deriving
 *                                       the 890 bytes per token"; "FP4 is a storage
 *                                       choice"]: E4M3FN bytes, one per 16 channels,
 *                                       scale = E4M3(max|x|/6), element = E2M1(x/scale);
 *                                       288 bytes per entry.  Other values of z_format
 *                                       return CSA2_ERR_UNSUPPORTED.
 *      ki_codes [B][entry_stride][64], ki_scales [B][entry_stride][4]   same format, 128 wide
 *      w_codes  [B][cap][512] E4M3FN, w_scale [B][cap] fp32: window ring, the
 *               row of position p lives in slot p mod cap.
 *  - Rotary table: rope_cos, rope_sin fp32 [rope_rows][32]; row p holds the
 *    cos/sin of the 32 angles of position p (pairs (lo+2i, lo+2i+1)).
 *  - Device-resident integers (positions, entry counts, indices) cannot be
 *    checked without a synchronisation.  Kernels clamp every one of them into
 *    its buffer, so a wrong value gives wrong numbers but never an access out
 *    of bounds.  Host-visible sizes are validated before anything is launched:
 *    on failure the call returns a status, launches nothing, writes nothing
 *    and records a message for csa2_last_error().
 *  - A call with no work (T, Tq or rows = 0; B = 0 for csa2_append) returns
 *    CSA2_OK after the size checks, reads no pointer and launches nothing.
 *  - No C++ exception crosses this boundary.  Calls are thread-safe.
 *
 * Citations name the page and the passage that defines each operation:
 *  [atlas]  "DeepSeek V4.1 -- Pooled group -> Source layer, pairs pooled"
 *           (equations of compressed sparse attention; cache note "between
 *           forward calls").
 *  [norm]   "DeepSeek V4.1 -- Window layer -> Attention RMSNorm".
 *  [blog]   "Inside DeepSeek V4.1", sections "Attention that looks at 640
 *           places" and "890 bytes".
 *  [zharf]  "Inside DeepSeek V4.1 Flash: Deriving the 890-Byte KV Cache",
 *           sections "Deriving the 890 bytes per token", "FP4 is a storage
 *           choice", the CSA2 section and "Bounded replay trades exact state
 *           for cheaper resumption".
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_ABI_VERSION 3

typedef enum {
    CSA2_OK = 0,
    CSA2_ERR_NULL = 1,        /* a required pointer is NULL */
    CSA2_ERR_SHAPE = 2,       /* a size is negative or inconsistent */
    CSA2_ERR_UNSUPPORTED = 3, /* a size the kernels do not implement (e.g. heads not a multiple of 16) */
    CSA2_ERR_RANGE = 4,       /* a buffer is too small for the stated sizes (ring, rotary table, cache) */
    CSA2_ERR_WORKSPACE = 5,   /* workspace missing or smaller than csa2_workspace_size() */
    CSA2_ERR_HIP = 6          /* the HIP runtime reported an error at launch */
} csa2_status;

/* workspace query ops */
#define CSA2_OP_INDEX_TOPK 1
#define CSA2_OP_SPARSE_ATTN 2
#define CSA2_OP_FORWARD 3
#define CSA2_OP_INDEX_SCORES 4
#define CSA2_OP_INDEX_POOL 5
#define CSA2_OP_REINDEX 6

/*
 * Compression of new positions into the compressed cache and the index-key
 * cache [atlas: k^p = sum_i softmax_i(g^c_i) (.) k^c_i over i in {2j, 2j+1};
 * c = gamma_C (.) k^p / sqrt(mean(k^p^2) + eps) with eps = 1e-20 [norm];
 * Z_{j,448:} <- R_{2j} c_{j,448:}; Z <- FP4(Z); k^i = c W_IK; k^n = RMSNorm;
 * K^I_{j,64:} <- R_{2j} k^n_{j,64:}; K^I <- FP4(K^I)].
 *
 *  B, T      requests, new positions per request (T >= 0; floor(T/ratio)
 *            entries are written; at ratio 2 an odd last position is left
 *            for the caller).
 *  pos0      [B] int32 device: absolute position of each request's first new
 *            token; even at ratio 2.  Entry j = pos0/ratio + i is written at
 *            cache row j (rows >= entry_stride are skipped).
 *  kc, gc    [B][T][512] bf16: pooled keys and gate logits of the new tokens
 *            (gc is not read, and may be NULL, at ratio 1).
 *  gamma_c   [512] fp32 RMSNorm gain of the compressed rows.
 *  w_ik      [512][128] bf16 index-key projection, or NULL for given mode.
 *  gamma_ik  [128] fp32 gain of the index-key norm (derive mode only).
 *  ki_given  [B][T/ratio][128] bf16 given index keys (already normalised
 *            and rotated; only encoded), used when w_ik == NULL.
 *  rope_*    rotary table, rope_rows >= 1.
 *  outputs   z_codes, z_scales, ki_codes, ki_scales as described above.
 */
csa2_status csa2_compress(int B, int T, const int32_t* pos0, const uint16_t* kc,
                          const uint16_t* gc, const float* gamma_c, const uint16_t* w_ik,
                          const float* gamma_ik, const uint16_t* ki_given, const float* rope_cos,
                          const float* rope_sin, int64_t rope_rows, uint8_t* z_codes,
                          uint8_t* z_scales, uint8_t* ki_codes, uint8_t* ki_scales,
                          int64_t entry_stride, int ratio, int z_format, void* stream);

/*
 * Window rows [atlas: W_{t,448:} <- R_t w^n_{t,448:}; W <- FP8(W); blog: the
 * window is stored in FP8].  Row i of request b is the window vector of
 * position pos0[b] + i; it is rotated at that position and written to ring
 * slot (position mod cap) as E4M3FN codes with one fp32 scale (max|x|/448).
 *  wn  [B][T][512] bf16.   cap >= 1.
 */
csa2_status csa2_encode_window(int B, int T, const int32_t* pos0, const uint16_t* wn,
                               const float* rope_cos, const float* rope_sin, int64_t rope_rows,
                               uint8_t* w_codes, float* w_scale, int cap, void* stream);

/*
 * Decode append: one new token per request [atlas, cache note "between
 * forward calls": the window ring of 128 slots, the compressed and index-key
 * rows of the pairs seen so far, and the pooling source's pair buffer of two
 * tensors (pooled keys, gate logits) of 512].  For request b the token at
 * absolute position p = pos[b]:
 *   - its window vector is rotated at p and written to ring slot p mod cap,
 *     as csa2_encode_window does;
 *   - p even: the token opens pair p/2; its pooled key and gate logits are
 *     copied to the pair buffer (pair_kc[b], pair_gc[b]) and no entry is written;
 *   - p odd: the token closes pair j = p/2 with the token held in the pair
 *     buffer; entry j is computed from (buffer, new token) exactly as
 *     csa2_compress computes it from two tokens of one call, so appending
 *     tokens one at a time writes the same bytes as compressing them together.
 *     Rows j >= entry_stride are skipped.
 *   - ratio 1: every token writes its own entry j = p (and its window row);
 *     the pair buffer and gc are not used and may be NULL.
 *  pos        [B] int32 device, >= 0 (a negative position skips the request).
 *  kc, gc, wn [B][512] bf16: the new token's pooled key, gate logits, window vector.
 *  pair_kc, pair_gc [B][512] bf16 device, caller-owned state carried between
 *             calls.  After a prefill of odd length the caller seeds them
 *             with the last token's kc and gc (or appends that token here).
 *  ki_given   [B][128] bf16 given index key of the entry the token writes: at
 *             ratio 2 the entry an odd token closes (read only for odd
 *             positions), at ratio 1 the token's own; only when w_ik == NULL.
 *  Other arguments as for csa2_compress and csa2_encode_window.  Requests
 *  are independent; two calls on one stream are ordered, so the pair buffer
 *  written by one call is read by the next.
 */
csa2_status csa2_append(int B, const int32_t* pos, const uint16_t* kc, const uint16_t* gc,
                        const uint16_t* wn, uint16_t* pair_kc, uint16_t* pair_gc,
                        const float* gamma_c, const uint16_t* w_ik, const float* gamma_ik,
                        const uint16_t* ki_given, const float* rope_cos, const float* rope_sin,
                        int64_t rope_rows, uint8_t* z_codes, uint8_t* z_scales,
                        uint8_t* ki_codes, uint8_t* ki_scales, int64_t entry_stride, int ratio,
                        int z_format, uint8_t* w_codes, float* w_scale, int cap, void* stream);

/*
 * Lightning indexer and causal top-512 [atlas: S^I_{t,j} = sum_h w^I_{t,h}
 * ReLU(Q^I_{h,t} . K^I_j); I_t = top_512(S^I_{t,j} : j < floor((t+1)/2)), with
 * the entries' ratio in place of 2;
 * blog: 32 heads of 128, one key per entry].
 *  Tq        query tokens per request, at positions q_pos0[b] + i.
 *  q_pos0    [B] int32 device.   n_entries [B] int32 device: valid cache rows.
 *  qI        [B][Tq][32][128] bf16 index queries (already rotated); each
 *            (token, head) row is quantised to E4M3FN with scale max|x|/448.
 *  wI        [B][Tq][32] fp32 head weights (the 1/sqrt(128*32) already applied).
 *  idx       [B][Tq][512] int32 out: chosen entries in ascending order,
 *            padded with -1.  Ties: larger score, then smaller entry.
 *  cnt       [B][Tq] int32 out: min(512, min(floor((p+1)/ratio), n_entries)).
 *  ws        workspace of at least csa2_workspace_size(CSA2_OP_INDEX_TOPK, ...).
 */
csa2_status csa2_index_topk(int B, int Tq, const int32_t* q_pos0, const int32_t* n_entries,
                            const uint16_t* qI, const float* wI, const uint8_t* ki_codes,
                            const uint8_t* ki_scales, int64_t entry_stride, int ratio,
                            int32_t* idx, int32_t* cnt, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * csa2_index_topk without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * csa2_index_topk; its scratch is one array of CSA2_NOALLOC_SCRATCH_BYTES
 * inside the library, one per GPU, held until the process ends (its address is
 * looked up once per device, with that device current, on the first call).
 * Sizes whose workspace (csa2_workspace_size(CSA2_OP_INDEX_TOPK, ...)) exceeds
 * it return CSA2_ERR_WORKSPACE.  Every call on a GPU uses that GPU's one array
 * and leaves its contents behind: two calls that overlap on one GPU (other
 * streams, other threads) race and give wrong results; calls ordered on one
 * stream are safe.  The current device must be the one `stream` belongs to.
 */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
csa2_status csa2_index_topk_noalloc(int B, int Tq, const int32_t* q_pos0,
                                    const int32_t* n_entries, const uint16_t* qI,
                                    const float* wI, const uint8_t* ki_codes,
                                    const uint8_t* ki_scales, int64_t entry_stride, int ratio,
                                    int32_t* idx, int32_t* cnt, void* stream);

/*
 * Full-layer selection plus the hierarchical candidate pool [blog: the
 * Hierarchical Sparse Indexer paragraph; zharf: section "Hierarchical indexing
 * bounds the later searches"].  idx and cnt exactly as csa2_index_topk.  From
 * the same scores, each query's candidates j < n are cut into blocks of 8
 * (block k = entries 8k..8k+7, the last may be short) keyed by their largest
 * score; the pool holds the block with the newest entry (n-1) and the 2,047
 * other blocks with the largest keys (ties: the smaller block), i.e. every
 * block when there are at most 2,048: at most 16,384 candidates.
 *  pool      [B][Tq][2048] int32 out: pool blocks in ascending order, -1 padded.
 *  pool_cnt  [B][Tq] int32 out: number of pool blocks, min(2048, ceil(n/8)).
 *  ws        at least csa2_workspace_size(CSA2_OP_INDEX_POOL, ...) bytes.
 */
csa2_status csa2_index_pool(int B, int Tq, const int32_t* q_pos0, const int32_t* n_entries,
                            const uint16_t* qI, const float* wI, const uint8_t* ki_codes,
                            const uint8_t* ki_scales, int64_t entry_stride, int ratio,
                            int32_t* idx, int32_t* cnt, int32_t* pool, int32_t* pool_cnt,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Reindex selection [same passages: a Reindex layer borrows the keys and the
 * pool, runs its own index query over the pool's candidates only, and takes
 * its own top 512].  Scores the entries of each query's pool blocks below n
 * with this layer's qI / wI against the shared ki cache (same arithmetic as
 * csa2_index_topk) and keeps the 512 largest (ties: smaller entry), in
 * ascending order, -1 padded; cnt = min(512, candidates).  The work per query
 * is bounded by the pool (16,384 candidates), not by the context.
 *  pool, pool_cnt  as written by csa2_index_pool for the same q_pos0 / n_entries.
 *  ws        at least csa2_workspace_size(CSA2_OP_REINDEX, ...) bytes.
 */
csa2_status csa2_reindex_topk(int B, int Tq, const int32_t* q_pos0, const int32_t* n_entries,
                              const uint16_t* qI, const float* wI, const uint8_t* ki_codes,
                              const uint8_t* ki_scales, int64_t entry_stride, int ratio,
                              const int32_t* pool, const int32_t* pool_cnt, int32_t* idx,
                              int32_t* cnt, void* ws, size_t ws_bytes, void* stream);

/*
 * The indexer's raw scores without selection [atlas: S^I_{t,j} = sum_h
 * w^I_{t,h} ReLU(Q^I_{h,t} . K^I_j)], same queries and keys as
 * csa2_index_topk.  scores [B][Tq][entry_stride] fp32: for query i of request
 * b only entries j < min(floor((p+1)/ratio), n_entries[b]) are written.
 *  ws  at least csa2_workspace_size(CSA2_OP_INDEX_SCORES, ...) bytes.
 */
csa2_status csa2_index_scores(int B, int Tq, const int32_t* q_pos0, const int32_t* n_entries,
                              const uint16_t* qI, const float* wI, const uint8_t* ki_codes,
                              const uint8_t* ki_scales, int64_t entry_stride, int ratio,
                              float* scores, void* ws, size_t ws_bytes, void* stream);

/*
 * Sparse shared-latent attention with a sink [atlas: J^w_t = {max(0,t-127)..t};
 * Y = [W; Z]; J = [J^w; I + |W|]; G_t = Y[J_t]; S = Q . G / sqrt(512);
 * A = exp S / (exp s_h + sum exp S); O = sum A G; O_{448:} <- R_t^{-1} O_{448:};
 * blog: one key-value vector per place shared by all heads, per-head sink].
 *  H         query heads, a multiple of 16 in 16..64.
 *  Q         [B][H][Tq][512] bf16, already rotated.
 *  cap       window ring capacity, >= Tq + 127 and at most 8388607;
 *            entry_stride at most 16777215 (CSA2_ERR_RANGE otherwise).
 *  idx, cnt  as produced by csa2_index_topk.
 *  sink      [H] fp32.
 *  O         [B][H][Tq][512] bf16 out.   lse [B][H][Tq] fp32 out or NULL
 *            (natural log of the full softmax denominator, sink included).
 *  z_format  storage of z_codes / z_scales (see the cache layout above).  With
 *            z_format 1 the rows are dequantised to bf16 before both products
 *            (the MFMA's scale operand is one power of two per 32 elements).
 *  win_floor [B] int32 device or NULL: bounded replay [zharf, section
 *            "Bounded replay trades exact state for cheaper resumption": for
 *            replay starting at s, a query at p sees window positions
 *            max(s, p-127) .. p].  s > p is read as s = p.
 */
csa2_status csa2_sparse_attn(int B, int Tq, int H, const int32_t* q_pos0, const uint16_t* Q,
                             const uint8_t* w_codes, const float* w_scale, int cap,
                             const uint8_t* z_codes, const uint8_t* z_scales, int64_t entry_stride,
                             int z_format, const int32_t* idx, const int32_t* cnt,
                             const float* sink, const float* rope_cos, const float* rope_sin,
                             int64_t rope_rows, uint16_t* O, float* lse, const int32_t* win_floor,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * The whole layer for one call [atlas, the compressed-sparse-attention
 * equations in order: pooling of pairs, compressed RMSNorm, rotation at 2j and
 * FP4 storage of Z and K^I; the FP8 window; the indexer score and the causal
 * top-512; the gather of window and selected rows; the sink softmax; the
 * inverse rotation of the output; blog, "Attention that looks at 640 places"].
 *  Prefill (kc != NULL): compress the T new positions (at pos0[b] .. pos0[b]+T-1,
 *  pos0 even at ratio 2; entries below pos0/ratio are the caches' earlier
 *  contents), write their window rows, then select and attend for every new
 *  position; n_entries may be NULL (then floor((pos0+T)/ratio) per request).
 *  Decode (kc == NULL): caches are given.  If wn != NULL the new tokens'
 *  window rows are written first.  n_entries is required.
 *  win_floor [B] int32 device or NULL: bounded replay, as for csa2_sparse_attn.
 *  Arguments as in the calls above; T is the number of query tokens.
 */
csa2_status csa2_forward(int B, int T, int H, const int32_t* pos0, const uint16_t* kc,
                         const uint16_t* gc, const uint16_t* wn, const float* gamma_c,
                         const uint16_t* w_ik, const float* gamma_ik, const uint16_t* ki_given,
                         const uint16_t* Q, const uint16_t* qI, const float* wI, const float* sink,
                         const float* rope_cos, const float* rope_sin, int64_t rope_rows,
                         uint8_t* z_codes, uint8_t* z_scales, uint8_t* ki_codes,
                         uint8_t* ki_scales, int64_t entry_stride, int ratio, int z_format,
                         const int32_t* n_entries, uint8_t* w_codes, float* w_scale, int cap,
                         int32_t* idx, int32_t* cnt, uint16_t* O, float* lse,
                         const int32_t* win_floor, void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace an op needs for these sizes (0 on invalid sizes). */
size_t csa2_workspace_size(int op, int B, int Tq, int H, int64_t entry_stride);

/*
 * Storage encoders used to fill caches from given values [zharf: E2M1 with
 * block scales; blog: FP8 window].  x [rows][cols] bf16.
 *  fp4: cols a multiple of 32; codes [rows][cols/2], scales [rows][cols/32].
 *  fp4e4 (the pages' format, z_format 1): cols a multiple of 16; codes
 *       [rows][cols/2], E4M3 scales [rows][cols/16].
 *  fp8: cols in 1..1024; codes [rows][cols], scale [rows] (max|x|/448, 1 if 0).
 */
csa2_status csa2_encode_fp4_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* codes,
                                 uint8_t* scales, void* stream);
csa2_status csa2_encode_fp4e4_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* codes,
                                   uint8_t* scales, void* stream);
csa2_status csa2_encode_fp8_rows(const uint16_t* x, int64_t rows, int cols, uint8_t* codes,
                                 float* scale, void* stream);

/*
 * The index queries as the indexer's matrix products take them [atlas:
 * indexer equation; the query rows quantised to FP8 for the FP8 x FP4
 * product].  Each (token, head) row of 128 bf16 values x gets the scale
 * s = max|x| / 448 (1 for an all-zero row) and the codes E4M3FN(x / s)
 * (fp32 division, nearest even, saturating); the row's head weight is folded
 * with its scale, wq = wI * s (one fp32 product).  The indexer's scoring
 * kernels quantise with the same device routine.
 *  qI [rows][128] bf16, wI [rows] fp32 -> q8 [rows][128] E4M3FN codes, wq [rows] fp32.
 */
csa2_status csa2_quant_index_query(const uint16_t* qI, const float* wI, int64_t rows, uint8_t* q8,
                                   float* wq, void* stream);

/* Dequantisation as the attention kernel performs it, to bf16 (exact for these formats). */
csa2_status csa2_decode_fp4_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                 int cols, uint16_t* out, void* stream);
csa2_status csa2_decode_fp4e4_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                   int cols, uint16_t* out, void* stream);
csa2_status csa2_decode_fp8_rows(const uint8_t* codes, int64_t rows, int cols, uint16_t* out,
                                 void* stream);

const char* csa2_status_string(csa2_status s);
const char* csa2_last_error(void);
int csa2_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
