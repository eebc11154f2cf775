/*
 * gqa_attn.h -- C ABI of an MI355X (gfx950) library for Gemma-4-style
 * grouped-query attention over a KV cache.
 *
 * The method (TensorFold pull-request pages):
 *   - PR #1183 "cuda gemma4: images on the 12B, and LayerNorm rows to 8192
 *     wide", squashed commit bodies, the window_rows notes: decode splits a
 *     head's keys into 256-key chunks, each leaving a partial (max, sum,
 *     accumulator), merged in chunk order; prompt tiles score over 128-dim
 *     slices; P may be kept to 16 bits as two bf16 halves; at head dim 512 no
 *     window applies, over a linear cache of up to 262144 keys, GQA 8 and 16.
 *   - PR #1183, same commit bodies, the Gemma 4 CUDA engine note: a sliding
 *     ring per sliding layer (window plus a chunk), a linear cache per global
 *     layer, prompt chunks of up to 512 rows; positions and slots of a decode
 *     forward are read on the device.
 *   - PR #975 "Gemma 4 12B on the native Metal engine", commit bodies: the
 *     cache is written before prompt attention, which takes its first new
 *     key from the metadata; 16-row query tiles under causal and sliding-
 *     window masks with an online softmax whose maxima and probabilities
 *     cross once a key block; value reads stop at the last written key.
 *   - PR #1184 "z-lab's DFlash drafter on the 31B", gotchas: the cache keeps
 *     a context's heads one capacity apart.
 *
 * Conventions for every call:
 *   - bf16 tensors are raw 16-bit patterns (uint16 storage), row-major.
 *   - Pointers marked "device" are device memory of the current HIP device;
 *     the library allocates nothing, keeps no state and is thread-safe.
 *   - `stream` is a hipStream_t passed as void*; NULL is the null stream.
 *     Every compute call only enqueues work on `stream` and returns.
 *   - Arguments are checked before anything is launched; a refusal returns
 *     a negative ATTN_E_* status and launches nothing.  A launch failure
 *     returns ATTN_E_LAUNCH.  No C++ exception crosses this interface.
 *   - Device-side values (decode positions) are trusted: they select which
 *     slots count, but every slot read lies inside [0, cache_cap) whatever
 *     they hold.
 *
 * Notation: S streams, Hq query heads, Hkv KV heads, G = Hq / Hkv query heads
 * per KV head (query head h uses KV head h / G), D head dim, cap cache slots.
 * Cache layout: [S][Hkv][cap][D] (decode) or [Hkv][cap][D] (one prompt
 * stream): heads cap apart.  Linear cache: slot j holds position j.  Ring of
 * cap slots: position p lives in slot p mod cap.
 * A row at position t attends key positions p with p <= t and, when the
 * window W > 0, t - p < W (the row itself and the W-1 before it).
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
enum {
    ATTN_OK = 0,
    ATTN_E_NULL = -1,        /* a required pointer is NULL                  */
    ATTN_E_HEAD_DIM = -2,    /* head_dim not 256 or 512                     */
    ATTN_E_GQA = -3,         /* Hq, Hkv < 1, Hq % Hkv != 0 or G > 16        */
    ATTN_E_WINDOW = -4,      /* window < 0, ring window > cap, or a prompt
                                ring with no window                         */
    ATTN_E_CACHE = -5,       /* cap < 1, or a prompt chunk that does not fit
                                (linear: pos0 + n_rows > cap; ring:
                                cap < window + n_rows - 1)                  */
    ATTN_E_ALIGN = -6,       /* a pointer not 16-byte aligned               */
    ATTN_E_WORKSPACE = -7,   /* decode workspace NULL or too small          */
    ATTN_E_P_MODE = -8,      /* unknown P mode, or one the call cannot take */
    ATTN_E_RANGE = -9,       /* a count < 0, pos0 < 0, non-finite scale, or
                                sizes whose byte offsets overflow 64 bits   */
    ATTN_E_LAUNCH = -10,     /* the HIP runtime refused a launch            */
    ATTN_E_UNSUPPORTED = -11 /* an argument reserved for a later extension  */
};

/* where softmax probabilities are rounded before they multiply V */
enum {
    ATTN_P_FP32 = 0,   /* not rounded (decode)                               */
    ATTN_P_BF16 = 1,   /* P = bf16(p)                                        */
    ATTN_P_BF16X2 = 2  /* P = bf16(p) + bf16(p - bf16(p)): two bf16 halves    */
};

/* slots per decode partial: the 256-key chunks of the window_rows note */
#define ATTN_DECODE_CHUNK 256

/*
 * Bytes of device workspace attn_decode needs: one fp32 partial
 * (max, sum, accumulator[D]) per (stream, query head, 256-slot chunk), the
 * scratch PR #975's decode notes size by the number of chunks, or per run
 * where runs are shorter than a chunk (caches of at most 1024 slots).
 * Returns 0 for arguments attn_decode would refuse.
 */
size_t attn_decode_workspace_bytes(int n_seq, int n_q_heads, int head_dim,
                                   int cache_cap);

/*
 * One decode row per stream (PR #1183 window_rows notes; PR #975 decode
 * attention commits).  For stream s and query head h, with t = pos[s]:
 * keys are the cache slots whose position is attended by a row at t; each
 * run c of consecutive slots (1 to 8 256-slot chunks, or a half or quarter
 * chunk in caches of at most 1024 or 512 slots: fixed by cap alone)
 * yields m_c (a reference maximum within 8 of the run's largest score, in
 * log2 units), l_c = sum 2^(s log2(e) - m_c) and acc_c = the same weights
 * times v (at head dim 256 the run's even and odd 32-slot blocks are summed
 * apart, each against its own reference maximum, and joined once); runs
 * merge in ascending order over M = max m_c; out =
 * bf16(sum e^(m_c - M) acc_c / sum e^(m_c - M) l_c).  Scores are scale * q.k
 * with fp32 accumulation; probabilities stay fp32, never rounded to bf16
 * (each enters the P.V products as three bf16 pieces whose sum is exactly
 * p).  A row's bits depend on neither n_seq nor the other streams.  This is
 * attn_decode_rows with one row per stream.  A row with no attended key
 * (t < 0) gives +0.
 *
 *   out        device bf16 [S][Hq][D], written
 *   q          device bf16 [S][Hq][D]
 *   k_cache    device bf16 [S][Hkv][cap][D]
 *   v_cache    device bf16 [S][Hkv][cap][D]
 *   pos        device int32 [S]: each stream's row position t
 *   n_seq      S >= 0 (0 launches nothing)
 *   ring       0 linear cache, 1 ring of cap slots
 *   window     W >= 0, 0 = none; a ring needs W <= cap
 *   cache_cap  cap >= 1, cap * D * 2 < 2^32 (one head's slice in 32-bit byte
 *              offsets), else ATTN_E_RANGE
 *   scale      finite fp32 score scale
 *   workspace  device, >= attn_decode_workspace_bytes(S, Hq, D, cap) bytes,
 *              16-byte aligned; contents on entry are ignored
 */
int attn_decode(void* out, const void* q, const void* k_cache,
                const void* v_cache, const int32_t* pos, int n_seq,
                int n_q_heads, int n_kv_heads, int head_dim, int cache_cap,
                int ring, int window, float scale, void* workspace,
                size_t workspace_bytes, void* stream);

/* Bytes of the library's own device array that attn_decode_noalloc keeps
   its partials in (one array per device, held until the process ends). */
#define ATTN_DECODE_SCRATCH_BYTES (16u << 20)

/*
 * attn_decode for callers that cannot allocate device memory: code that a
 * HIP graph captures, serving loops and harnesses that forbid hipMalloc.
 * The chunk-run partials go to a fixed array of ATTN_DECODE_SCRATCH_BYTES
 * inside the library instead of a caller's workspace; the call allocates
 * nothing and issues no memset.  Kernels, arithmetic and output bits are
 * attn_decode's.
 *
 * Arguments and errors as attn_decode, without the workspace, plus:
 *   ATTN_E_WORKSPACE  the partials do not fit the array: S * Hq * runs *
 *                     (D + 2) * 4 bytes > ATTN_DECODE_SCRATCH_BYTES, runs =
 *                     ceil(n / c), n = ceil(cap / 256) chunks, c = floor(n / 16)
 *                     clamped to 1..8 (e.g. 8 streams x 32 heads at D = 512
 *                     over 32768 keys, or one stream over 262144, use 8.4 MB)
 *   ATTN_E_LAUNCH     also when the array's device address cannot be found
 * Every call on a device shares that device's array, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls that may
 * overlap on one device (other streams, other host threads) race and must
 * be ordered by the caller.
 */
int attn_decode_noalloc(void* out, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* pos, int n_seq,
                        int n_q_heads, int n_kv_heads, int head_dim, int cache_cap,
                        int ring, int window, float scale, void* stream);

/* Largest decode window (rows per stream) of attn_decode_rows. */
#define ATTN_DECODE_MAX_ROWS 16

/*
 * Workspace bytes attn_decode_rows needs for these sizes (device memory the
 * caller allocates; partials of every row, head and chunk run).  Returns 0
 * for arguments attn_decode_rows would refuse.
 */
size_t attn_decode_rows_workspace_bytes(int n_seq, int rows, int n_q_heads,
                                        int head_dim, int cache_cap);

/*
 * Decode windows: `rows` consecutive rows per stream, row r of stream s at
 * position pos[s] + r (PR #975 decode attention commits: a key head's query
 * heads and two decode rows fill one 16-row tile, each key and value read
 * once for the window, and every row keeps its bits at any window width;
 * PR #1183 engine note: windows of up to 16 rows a stream).  Each row is an
 * ordinary decode row of its position (causal, window W): the keys are the
 * cache slots it attends, split into runs of slots (as attn_decode) whose partials
 * merge in ascending order over the largest run maximum.  Probabilities stay
 * fp32 (the P.V products take each p as three bf16 pieces whose sum is p
 * exactly).  A row's output depends neither on `rows` nor on n_seq nor on
 * which other rows share the call: rows = 1 gives attn_decode's bits.
 * Every row's own key and value must already be in the cache
 * (attn_cache_write of the window's rows first).
 *
 *   out        device bf16 [S][rows][Hq][D], written
 *   q          device bf16 [S][rows][Hq][D]
 *   k_cache    device bf16 [S][Hkv][cap][D]
 *   v_cache    device bf16 [S][Hkv][cap][D]
 *   pos        device int32 [S]: position of each stream's first row (read on
 *              the device, not checked; pos[s] + rows - 1 must fit in int32)
 *   n_seq      S >= 0 (0 launches nothing)
 *   rows       1 .. ATTN_DECODE_MAX_ROWS
 *   ring       0 linear cache, 1 ring of cap slots: then 1 <= W and
 *              W + rows - 1 <= cap, so the later rows' writes leave the
 *              first row's window in the ring
 *   window     W >= 0, 0 = none (linear only)
 *   scale      finite fp32 score scale
 *   workspace  device, >= attn_decode_rows_workspace_bytes(S, rows, Hq, D,
 *              cap) bytes, 16-byte aligned; contents on entry are ignored
 * Errors as attn_decode, plus ATTN_E_RANGE for rows outside 1..16 and
 * ATTN_E_WINDOW for a ring whose W is 0 or leaves fewer than rows - 1 spare
 * slots.
 */
int attn_decode_rows(void* out, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* pos, int n_seq, int rows,
                     int n_q_heads, int n_kv_heads, int head_dim, int cache_cap,
                     int ring, int window, float scale, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Bytes at the start of a fused decode's workspace that hold its counters. */
#define ATTN_DECODE_COUNTER_BYTES 262144

/*
 * attn_decode_rows in one launch where it can (PR #975 decode commits: with
 * one key chunk the partial writes the merged output itself, e^(top - top)
 * being 1; the Gemma 4 CUDA engine note in PR #1183: a decode forward's
 * launches depend on its row count alone, positions read on the device, so
 * each row count is captured once as a graph and replayed).  With one run
 * per (stream, KV head) the kernel writes the output directly; with up to 16
 * runs the last workgroup to finish merges, in the merge kernel's order;
 * beyond that it is attn_decode_rows (partials, then the merge).  Outputs
 * are bit for bit those of attn_decode_rows.  Nothing is allocated and no
 * memset is issued, so a graph may capture the call.
 *
 * Arguments as attn_decode_rows, except the workspace: at least
 * ATTN_DECODE_COUNTER_BYTES + attn_decode_rows_workspace_bytes(...) bytes,
 * whose first ATTN_DECODE_COUNTER_BYTES must be zero on entry (set once by
 * attn_decode_workspace_init; every call leaves them zero).  Calls that
 * share a workspace must not overlap.  ATTN_E_RANGE when n_seq * Hkv >
 * 4096 (the counter area's limit).
 */
int attn_decode_rows_fused(void* out, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* pos, int n_seq, int rows,
                           int n_q_heads, int n_kv_heads, int head_dim, int cache_cap,
                           int ring, int window, float scale, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Zeroes the counter area (first ATTN_DECODE_COUNTER_BYTES) of a workspace
 * for attn_decode_rows_fused, by a kernel on `stream`.  Needed once per
 * workspace, and again after the workspace served anything else.
 * ATTN_E_WORKSPACE for a NULL or smaller workspace, ATTN_E_ALIGN unless
 * 16-byte aligned.
 */
int attn_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode prologue of one stacked projection row per stream (PR #1183
 * squashed commit bodies, the qk_rows note: q and k = bf16(w * bf16(x *
 * inv)) before the rotary embedding, inv = 1 / sqrt(mean(x^2) + eps), and v
 * optionally normed by a unit RMS norm; PR #975 decode commits: the row's
 * key and value go to the cache).  For stream s at t = pos[s], each head's
 * D values x of q and k are normed with their scale (q_norm_w or k_norm_w,
 * two bf16 rounding points) and rotated over the head's halves: for
 * i < D/2, a = fp32(fp32(t) * inv_freq[i]), out_i = bf16(y_i cos a -
 * y_{i+D/2} sin a), out_{i+D/2} = bf16(y_{i+D/2} cos a + y_i sin a) (cos and
 * sin of the fp32 angle in fp32; a zero frequency leaves its pair as is).
 * v is bf16(x * inv) when v_norm = 1, else copied.  q goes to q_out; the
 * key and value to the cache slot of t (t, or t mod cap in a ring).
 *
 *   q_out      device bf16 [S][Hq][D], written
 *   k_cache    device bf16 [S][Hkv][cap][D], slot of pos[s] written
 *   v_cache    device bf16 [S][Hkv][cap][D], slot of pos[s] written
 *   qkv        device bf16 [S][(Hq + 2 Hkv) D]: q heads, k heads, v heads
 *   q_norm_w   device bf16 [D], 16-byte aligned
 *   k_norm_w   device bf16 [D], 16-byte aligned
 *   inv_freq   device fp32 [D/2]
 *   eps        finite, >= 0 (a zero row with eps = 0 gives NaN)
 *   v_norm     0 or 1
 *   pos        device int32 [S]; a row with t < 0, or t >= cap in a linear
 *              cache, writes no key or value
 * Errors as attn_decode for shapes; ATTN_E_RANGE for eps or v_norm.
 */
int attn_qkv_prep(void* q_out, void* k_cache, void* v_cache, const void* qkv,
                  const void* q_norm_w, const void* k_norm_w, const float* inv_freq, float eps,
                  int v_norm, const int32_t* pos, int n_seq, int n_q_heads, int n_kv_heads,
                  int head_dim, int cache_cap, int ring, void* stream);

/*
 * attn_qkv_prep followed by attn_decode_rows_fused with one row per stream,
 * in the decode kernel itself (PR #975 decode commits: the partial kernel
 * norms and ropes its query heads from the stacked row, the workgroup of
 * the row's chunk writes the row's key and value to the cache, and with one
 * chunk it writes the output itself).  Outputs, cache contents and bits are
 * those of the two calls.  Arguments as the two calls; the caches are
 * written; the workspace as attn_decode_rows_fused's (counters set up by
 * attn_decode_workspace_init).
 */
int attn_decode_prep_fused(void* out, const void* qkv, const void* q_norm_w,
                           const void* k_norm_w, const float* inv_freq, float eps, int v_norm,
                           void* k_cache, void* v_cache, const int32_t* pos, int n_seq,
                           int n_q_heads, int n_kv_heads, int head_dim, int cache_cap,
                           int ring, int window, float scale, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Prompt attention for one stream's chunk of n_rows rows at positions
 * pos0 .. pos0 + n_rows - 1 (PR #975 prompt attention commits; PR #1183
 * window_rows notes).  The chunk's own keys and values must already be in
 * the cache (attn_cache_write).  Each row attends its positions (causal,
 * sliding window W when W > 0) in blocks of KB = attn_prefill_key_block()
 * keys aligned to absolute positions, in ascending order: the running
 * maximum m moves once a block, p = exp(s - m), P = round(p) per p_mode is
 * what multiplies V, the row sum takes unrounded p, and
 * out = bf16(acc / sum).  Keys outside a tile's attended span are never
 * read into the products (a never-written V row cannot turn into NaN).
 *
 *   out       device bf16 [n_rows][Hq][D], written
 *   q         device bf16 [n_rows][Hq][D]
 *   k_cache   device bf16 [Hkv][cap][D]
 *   v_cache   device bf16 [Hkv][cap][D]
 *   pos0      position of the first row, >= 0, with pos0 + n_rows + 64 <=
 *             INT32_MAX (positions are 32-bit ints), else ATTN_E_RANGE
 *   n_rows    >= 0 (0 launches nothing)
 *   ring      0 linear (pos0 + n_rows <= cap), 1 ring (0 < W <= cap and
 *             cap >= W + n_rows - 1, so no row's keys are overwritten)
 *   cache_cap cap * D * 2 < 2^32 (one head's slice in 32-bit byte offsets),
 *             else ATTN_E_RANGE
 *   p_mode    ATTN_P_BF16 or ATTN_P_BF16X2
 *   last_key  NULL: each row's last key is its own position (causal).  Or
 *             device int32 [n_rows], 4-byte aligned: the last key position
 *             row r attends (PR #975 commit body: the prompt attention takes
 *             each row's last key, its own position for text rows; PR #1183
 *             body: an image's rows see each other on sliding layers through
 *             the last-key rows).  Each value is clamped to [pos0 + r,
 *             pos0 + n_rows - 1]: never fewer keys than causal, never a key
 *             the chunk has not written.  The window's first key stays
 *             pos0 + r - W + 1.  Values are read on the device, not checked.
 */
int attn_prefill(void* out, const void* q, const void* k_cache,
                 const void* v_cache, int pos0, int n_rows, int n_q_heads,
                 int n_kv_heads, int head_dim, int cache_cap, int ring,
                 int window, float scale, int p_mode,
                 const int32_t* last_key, void* stream);

/* Bytes of device workspace attn_prefill_ws may use for n_rows rows of
   n_q_heads heads (partials of up to four key ranges per row and head); 0
   for arguments it would refuse. */
size_t attn_prefill_workspace_bytes(int n_rows, int n_q_heads, int head_dim);

/*
 * attn_prefill with a workspace, for launches that one workgroup per
 * 16-row tile would leave mostly idle (a 128-row chunk of a sliding layer
 * takes 64 workgroups on a 256-CU chip).  At head dim 256 the library then
 * splits each tile's key blocks into up to four consecutive ranges on
 * workgroups of their own; a range after the first first forms the scores of
 * the blocks before it, so that its running maxima, and with them every
 * rounded P, equal the unsplit walk's (PR #975 prompt attention commits: the
 * maximum moves once a block, p rounded against it); each range leaves a
 * partial (maximum, row sum, accumulator) and a merge launch joins them in
 * range order, as decode joins its chunk partials (PR #1183 window_rows
 * notes).  Outputs
 * differ from attn_prefill's only by the order of fp32 additions.  The split
 * count depends on n_rows, Hq and Hkv alone.  At head dim 512, or with a NULL
 * workspace, this is attn_prefill.
 *
 *   workspace        device, 16-byte aligned, >= attn_prefill_workspace_bytes
 *                    (n_rows, Hq, D) bytes (else ATTN_E_WORKSPACE); contents
 *                    on entry are ignored; calls sharing one must not overlap
 *   (the rest as attn_prefill)
 */
int attn_prefill_ws(void* out, const void* q, const void* k_cache,
                    const void* v_cache, int pos0, int n_rows, int n_q_heads,
                    int n_kv_heads, int head_dim, int cache_cap, int ring,
                    int window, float scale, int p_mode,
                    const int32_t* last_key, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * Write a chunk's new keys and values into the cache before attention
 * (PR #975, the cache-before-attention commit): row r goes to the slot of
 * position pos0 + r (linear: pos0 + r < cap required; ring: (pos0 + r) mod
 * cap, and n_rows <= cap).  Bit copies, no rounding.
 *
 *   k_cache, v_cache  device bf16 [Hkv][cap][D], updated
 *   k, v              device bf16 [n_rows][Hkv][D]
 */
int attn_cache_write(void* k_cache, void* v_cache, const void* k,
                     const void* v, int pos0, int n_rows, int n_kv_heads,
                     int head_dim, int cache_cap, int ring, void* stream);

/*
 * A whole prompt through one layer, in chunks (PR #975 commits: the prompt is
 * fed in chunks, and a chunk's keys and values enter the cache before its
 * attention reads them): rows r0 .. r0 + m - 1 of each chunk of `chunk` rows
 * (the last may be shorter) are attended as attn_prefill attends them after
 * attn_cache_write has put them in the cache.  The outputs and the final
 * cache are bit for bit those of attn_cache_write + attn_prefill chunk by
 * chunk.  Key blocks sit on absolute positions, so a row's bits do not depend
 * on the chunks, and the library attends the whole prompt in one launch:
 * into a linear cache every row is written first; with a ring, where chunk c
 * + 1 would overwrite keys chunk c still reads, the keys the prompt attends
 * (the window before pos0 from the ring, the prompt's own from k and v) go
 * to a linear copy in the workspace -- or, when the prompt attends no key
 * before pos0 (pos0 = 0, or a window of one) at head dim 256, are read in
 * place from k and v, leaving the workspace untouched -- and the prompt's
 * last rows enter the ring after the attention.
 *
 *   out, q            device bf16 [n_rows][Hq][D]
 *   k, v              device bf16 [n_rows][Hkv][D], the prompt's keys and
 *                     values (rotated, normed), row r at position pos0 + r
 *   k_cache, v_cache  device bf16 [Hkv][cap][D], written (and read)
 *   chunk             rows per chunk, >= 1 (else ATTN_E_RANGE); every chunk
 *                     must meet attn_prefill's conditions (a ring: cap >= W +
 *                     min(chunk, n_rows) - 1; a linear cache: pos0 + n_rows
 *                     <= cap, else ATTN_E_CACHE)
 *   last_key          NULL, or device int32 [n_rows]: as attn_prefill takes
 *                     it chunk by chunk (each value clamped to the last row of
 *                     its row's chunk)
 *   workspace         ring: device, 16-byte aligned, >=
 *                     attn_prefill_prompt_workspace_bytes(...) bytes (else
 *                     ATTN_E_WORKSPACE), contents ignored; a linear cache
 *                     needs none (NULL)
 *   (the rest as attn_prefill)
 */
size_t attn_prefill_prompt_workspace_bytes(int pos0, int n_rows, int n_kv_heads, int head_dim,
                                           int ring, int window);
int attn_prefill_prompt(void* out, const void* q, const void* k, const void* v,
                        void* k_cache, void* v_cache, int pos0, int n_rows, int chunk,
                        int n_q_heads, int n_kv_heads, int head_dim, int cache_cap, int ring,
                        int window, float scale, int p_mode, const int32_t* last_key,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The key block KB attn_prefill uses for (head_dim, p_mode): the block at
 * which the running maximum moves and P is rounded, which decides P's
 * rounded values.  64 at head dim 256, 32 at head dim 512.  Returns a
 * negative status for a head dim or P mode attn_prefill refuses.
 */
int attn_prefill_key_block(int head_dim, int p_mode);

/* Static, NUL-terminated name of a status code ("ATTN_OK", ...). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
