/*
 * pagedattn.h -- C ABI of a paged grouped-query attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * One operation in four call shapes: attention of a step's query rows over a
 * paged K/V cache -- the decode step (many sequences, one row each), the
 * speculative verify round (exactly eight rows per sequence, causal within
 * the round), and the prefill chunk (one sequence, many rows) -- with a bf16
 * or an fp8-e4m3 K/V cache, plus the append/quantise step that writes a
 * call's new K/V rows into the cache and a host-side block-table builder.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers unless the argument name ends in `_host`.
 *    The caller allocates and owns every buffer, including the workspace;
 *    the library allocates no device memory at run time.  State kept
 *    between calls: a per-thread error string; a per-device launch shape
 *    read once from the driver; the scratch array of
 *    attn_paged_decode_noalloc (part of the library's device code, one per
 *    GPU) and its address per GPU; and the two measurement hooks at the end
 *    of this header (a per-thread event pair consumed by the next call, and
 *    a process-wide grid bound that is 0, i.e. off, unless set).
 *  - Device work is enqueued on `stream` and is asynchronous: inputs must
 *    stay unchanged and outputs unread until the stream has passed the call.
 *    Outputs never alias inputs.
 *  - Return value: ATTN_OK, or a negative ATTN_E_* code.  Every argument the
 *    host can see is checked before anything is enqueued; on error nothing
 *    is written and attn_last_error() names the offending argument.  This
 *    follows "Radiance Architecture Plugins -- declaring a model", section
 *    "Step: issuing the graph": an op over zero rows is a shape error that
 *    writes nothing, and a failing helper sets a named status.
 *  - A shape or format the kernels do not serve returns ATTN_E_UNSUPPORTED;
 *    there is never a silent fallback to another path (same page, section
 *    "Probe: what the plugin measured": a switch that cannot be honoured is
 *    refused, never substituted).
 *  - head_dim is always an argument and is never computed from other sizes
 *    (same page, section "Declare: the metadata").
 *
 * Device-resident inputs (lengths, block tables) cannot be checked on the
 * host.  The kernels never read outside the buffers the sizes describe:
 *  - a sequence whose ctx_len is below the call's rows or above
 *    max_pages_per_seq * page_size gets NaN in every output element of its
 *    rows;
 *  - a block-table entry that a row needs and that lies outside
 *    [0, n_pages) is not dereferenced, and the rows that need it get NaN.
 * Callers that hold host copies may run attn_check_lengths_host() and
 * attn_check_block_table_host() first for a named error instead.
 *
 * Data layout
 * -----------
 *   Q / out            bf16 [n_seq][rows][n_head][head_dim], rows = 1 for
 *                      decode, 8 for verify; [n_rows][n_head][head_dim] for
 *                      prefill.
 *   k_pool / v_pool    [n_pages][n_head_kv][page_size][head_dim] of bf16, or
 *                      of e4m3 codes (one byte each) for ATTN_KV_FP8_E4M3.
 *                      One call covers one layer's pool.  The page count is
 *                      the caller's ("kern manifest v7" schema,
 *                      $defs.HostTensor: only the outermost extent is the
 *                      host's choice).
 *   k_scale / v_scale  fp32 [n_pages][n_head_kv]: one scale per page and kv
 *                      head, separately for K and V (fp8 only; NULL for bf16).
 *                      The stored value of element i is code_value * scale.
 *   block_table        int32 [n_seq][max_pages_per_seq]; token t of sequence
 *                      s lives in page block_table[s][t / page_size] at slot
 *                      t % page_size ("kern manifest v7" schema, $defs.Domain:
 *                      a block table whose index covers `stride` = 16 token
 *                      slots).  Entries past a sequence's last page are
 *                      never read.
 *   ctx_lens           int32 [n_seq]: each sequence's length AFTER this call,
 *                      i.e. the rows already cached plus this call's rows
 *                      (same schema, $defs.Fill "seq_len").  The call's K/V
 *                      must already be in the cache (attn_kv_append first).
 *                      Row r of a call with R rows sits at position
 *                      ctx_len - R + r and attends to keys 0 .. that position.
 *
 * Arithmetic: softmax(Q K^T / sqrt(head_dim)) V with fp32 accumulation,
 * bf16 output rounded to nearest-even.  GQA: query head h reads kv head
 * h / (n_head / n_head_kv).
 *
 * Determinism: decode and verify results depend only on the sequence's own
 * inputs -- never on the batch size, the other sequences, the order of the
 * batch or the device's compute-unit count -- and each verify row is bit for
 * bit the decode result for the same position over the same cache, as the
 * pages ask of a speculative round ("TandemLLM -- Adding a model", section
 * "The adapter path in ten steps", step 4).
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_KV_BF16 = 0, ATTN_KV_FP8_E4M3 = 1 } attn_kv_dtype;

enum {
    ATTN_OK = 0,
    ATTN_E_ARG = -1,         /* null pointer, negative size, bad enum           */
    ATTN_E_SHAPE = -2,       /* zero rows or sequences, heads not divisible ... */
    ATTN_E_UNSUPPORTED = -3, /* head_dim / page size / group size not served    */
    ATTN_E_WORKSPACE = -4,   /* workspace too small or misaligned               */
    ATTN_E_RANGE = -5,       /* host-checked length or table entry out of range */
    ATTN_E_DEVICE = -6       /* the HIP runtime refused a launch                */
};

/* Rows per sequence of a verify round: exact, not a bound ("kern manifest
   v7" schema, $defs.Batch: rows is 1 for a decode step and 8 for a
   speculative round). */
#define ATTN_VERIFY_ROWS 8

/* Page (block) size the kernels are built for.  The pages make the block
   size a property of the attention kernel, read back by the engine
   ("Radiance Architecture Plugins -- declaring a model", section "Declare:
   buffers and KV groups"); the schema's block-table example uses 16. */
#define ATTN_PAGE_SIZE 16

/*
 * attn_paged_decode -- one query row per sequence (decode step).
 *
 *   q          bf16 [n_seq][n_head][head_dim]
 *   out        bf16 [n_seq][n_head][head_dim]
 *   workspace  device scratch of at least
 *              attn_paged_workspace_bytes(0, n_seq, max_pages_per_seq,
 *              n_head, head_dim), 256-byte aligned; its contents are dead
 *              between calls ("kern manifest v7" schema, $defs.BufferKind
 *              "workspace").
 * Other arguments as described in the header comment.  Needs
 * n_head % n_head_kv == 0, n_head / n_head_kv <= 16, head_dim in {128, 256},
 * page_size == ATTN_PAGE_SIZE, n_seq <= 4096.
 */
int attn_paged_decode(const void* q, const void* k_pool, const void* v_pool,
                      const float* k_scale, const float* v_scale, int64_t n_pages,
                      const int32_t* block_table, int32_t max_pages_per_seq,
                      const int32_t* ctx_lens, int32_t n_seq, int32_t n_head,
                      int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                      attn_kv_dtype kv_dtype, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * attn_paged_verify -- exactly ATTN_VERIFY_ROWS query rows per sequence, the
 * round's draft tokens, causal within the round and after the cached context.
 *
 *   q, out     bf16 [n_seq][ATTN_VERIFY_ROWS][n_head][head_dim]
 *   workspace  attn_paged_workspace_bytes(1, ...)
 * Row r of sequence s is at position ctx_lens[s] - 8 + r; its result equals,
 * bit for bit, attn_paged_decode of that row with ctx_len = position + 1 over
 * the same cache.  Needs ctx_lens[s] >= 8 and, besides the decode limits,
 * ceil(8 / floor(16 / g)) * head_dim <= 512 with g = n_head / n_head_kv.
 */
/*
 * attn_paged_decode_noalloc -- attn_paged_decode without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).
 *
 * The split partials go to a scratch array inside the library (64 MiB, one
 * per GPU the library runs on, held until the process ends); the call makes
 * no allocation of any kind.  The caller still passes every input and the
 * output.  Arguments, limits and results are those of attn_paged_decode
 * (the same kernels: every output row is bit for bit attn_paged_decode's),
 * and additionally the call's partials,
 * attn_paged_workspace_bytes(0, n_seq, max_pages_per_seq, n_head, head_dim)
 * bytes, must fit the scratch array, else ATTN_E_WORKSPACE and nothing is
 * written.  All calls on one GPU share the array: calls that may overlap on
 * a GPU (several streams, several threads) race and must be serialised by
 * the caller.  Nothing in the array needs clearing between calls.
 */
int attn_paged_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                              const float* k_scale, const float* v_scale, int64_t n_pages,
                              const int32_t* block_table, int32_t max_pages_per_seq,
                              const int32_t* ctx_lens, int32_t n_seq, int32_t n_head,
                              int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                              attn_kv_dtype kv_dtype, void* out, hipStream_t stream);

int attn_paged_verify(const void* q, const void* k_pool, const void* v_pool,
                      const float* k_scale, const float* v_scale, int64_t n_pages,
                      const int32_t* block_table, int32_t max_pages_per_seq,
                      const int32_t* ctx_lens, int32_t n_seq, int32_t n_head,
                      int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                      attn_kv_dtype kv_dtype, void* out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * attn_paged_verify_width -- a speculative round of `width` rows per sequence,
 * 1 <= width <= ATTN_VERIFY_ROWS, causal within the round and after the
 * cached context ("TandemLLM -- Adding a model", section "The adapter path
 * in ten steps": a recorded decode is replayed as chains of every verify
 * width and every row must match bit for bit).
 *
 *   q, out     bf16 [n_seq][width][n_head][head_dim]
 *   workspace  attn_paged_workspace_bytes(1, ...) covers every width
 * Row r of sequence s is at position ctx_lens[s] - width + r; its result
 * equals, bit for bit, attn_paged_decode of that row with ctx_len =
 * position + 1 over the same cache (width 8 is attn_paged_verify, width 1
 * is attn_paged_decode).  Needs ctx_lens[s] >= width and, besides the
 * decode limits, ceil(width / floor(16 / g)) * head_dim <= 512 after
 * rounding the tile count up to 1, 2 or 4.
 */
int attn_paged_verify_width(const void* q, const void* k_pool, const void* v_pool,
                            const float* k_scale, const float* v_scale, int64_t n_pages,
                            const int32_t* block_table, int32_t max_pages_per_seq,
                            const int32_t* ctx_lens, int32_t n_seq, int32_t width,
                            int32_t n_head, int32_t n_head_kv, int32_t head_dim,
                            int32_t page_size, attn_kv_dtype kv_dtype, void* out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_paged_verify_tree -- a speculative round of `width` rows shaped as a
 * tree ("Radiance Architecture Plugins -- declaring a model", section
 * "Declare: drafters, encoders, generators": a drafter may propose a tree;
 * "TandemLLM -- Adding a model", section "The adapter path in ten steps":
 * rounds replayed as trees must match the recorded decode bit for bit).
 *
 *   q, out         bf16 [n_seq][width][n_head][head_dim]; the round's rows
 *                  are in the cache at positions C0 .. C0 + width - 1,
 *                  C0 = ctx_lens[s] - width (attn_kv_append first)
 *   tree_mask      int32 [n_seq][width], DEVICE: bit j of row r's entry set
 *                  = row r attends round row j.  A row names itself and only
 *                  earlier rows (its ancestors); anything else gives NaN rows.
 *   scratch_pages  int32 [n_seq][width][2], DEVICE: pool pages the call may
 *                  overwrite (two per row, distinct, unused by any sequence);
 *                  the branch views are built there.  With an fp8 pool their
 *                  scales are overwritten too.
 *   k_pool, v_pool, k_scale, v_scale  writable (scratch pages only).
 *   workspace      attn_paged_workspace_bytes(4, n_seq, ...)
 * Row r attends keys 0 .. C0 - 1 and the round rows its mask names, in row
 * order; its result equals, bit for bit, attn_paged_decode of the same row
 * over a cache holding the context followed by those rows at positions C0,
 * C0 + 1, ... (its branch).  A chain mask (row r names 0 .. r) gives the
 * attn_paged_verify_width rows.  bf16 bytes are copied into the views.
 * With an fp8 pool a view page takes the scale of the cache page holding its
 * first token and that page's codes; rows that move down into it from the
 * next page (a round across a page boundary whose branch skips rows) are
 * written as attn_kv_append would write them there at a later call: each
 * value (code times its page's scale, fp32) is encoded at the view page's
 * scale, doubled first while those values exceed 448 times it (the page's
 * other codes are then re-encoded too).  Needs n_seq * width <=
 * 4096 and at most 16 query heads per kv head.  The context below the
 * split holding C0 (splits of 1024 keys with an fp8 cache at head_dim 128,
 * else 512) is read once for all rows of a sequence (as by
 * attn_paged_verify_width); that split and the next are read per row.
 * Where attn_paged_verify_width would not serve `width` rows (its tile
 * limit), every row reads its whole context instead; the results are the
 * same bits.
 */
int attn_paged_verify_tree(const void* q, void* k_pool, void* v_pool, float* k_scale,
                           float* v_scale, int64_t n_pages, const int32_t* block_table,
                           int32_t max_pages_per_seq, const int32_t* ctx_lens, int32_t n_seq,
                           int32_t width, const int32_t* tree_mask, const int32_t* scratch_pages,
                           int32_t n_head, int32_t n_head_kv, int32_t head_dim,
                           int32_t page_size, attn_kv_dtype kv_dtype, void* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_paged_prefill -- a chunk of n_rows new rows of ONE sequence over its
 * cached context ("kern manifest v7" schema, $defs.Batch: rows given by the
 * chunk, one sequence; `context` is the cached rows it expands over).
 *
 *   q, out       bf16 [n_rows][n_head][head_dim]
 *   block_table  int32 [max_pages_per_seq] (the sequence's row)
 *   ctx_len      HOST value: the sequence's length after this call; row r is
 *                at position ctx_len - n_rows + r.  Checked on the host:
 *                n_rows <= ctx_len <= max_pages_per_seq * page_size.
 *   workspace    attn_paged_workspace_bytes(2, ...) (may be 0 bytes)
 * Needs n_head % n_head_kv == 0, head_dim in {128, 256}, kv_dtype bf16 or
 * fp8 (fp8 pages are dequantised to bf16 in registers).
 */
int attn_paged_prefill(const void* q, int32_t n_rows, const void* k_pool, const void* v_pool,
                       const float* k_scale, const float* v_scale, int64_t n_pages,
                       const int32_t* block_table, int32_t max_pages_per_seq, int32_t ctx_len,
                       int32_t n_head, int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                       attn_kv_dtype kv_dtype, void* out, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* prefill_fp8 bits of attn_paged_prefill_fp8. */
#define ATTN_PREFILL_FP8_QK 1
#define ATTN_PREFILL_FP8_PV 2

/*
 * attn_paged_prefill_fp8 -- attn_paged_prefill with the fp8 switch the
 * attention op carries ("Radiance Architecture Plugins -- declaring a
 * model", section "Declare: the metadata": the build context's
 * `attn_prefill_fp8` bits are passed as the op's `prefill_fp8`).  The pages
 * do not define the bits; here:
 *
 *   0                    attn_paged_prefill, bit for bit.
 *   ATTN_PREFILL_FP8_QK  (fp8 cache only) QK^T runs on the fp8 matrix unit:
 *                        K with its stored E4M3 codes and page scale, and
 *                        each query vector (one row, one head) rounded to
 *                        E4M3 at the smallest power-of-two scale 2^e with
 *                        max|q| <= 448 * 2^e (e >= -117), ties to even.
 *                        Softmax and PV are as in attn_paged_prefill.
 *   ATTN_PREFILL_FP8_PV  (fp8 cache only) PV runs on the fp8 matrix unit:
 *                        V with its stored E4M3 codes; each key tile's
 *                        (32 keys with both bits at head_dim 128 or 256 and
 *                        g dividing 128, else 64) probabilities p
 *                        (relative to the row's running
 *                        maximum, p <= 2^8) times its pages' V scales over
 *                        2^F -- F the exponent of the tile's largest V scale,
 *                        so the factors lie in (0, 1] -- rounded to E4M3
 *                        (nearest, ties to even); the products accumulate in
 *                        fp32 and are scaled by 2^F; the row sum is of the
 *                        unrounded p.  Each weight thus carries a relative
 *                        error of at most 2^-4 (E4M3 normals), so an output
 *                        element moves by at most 2^-4 times the same
 *                        softmax average of |v|: far below the fp8
 *                        tolerance over long contexts, up to about 6% of
 *                        |v| over a handful of keys.
 *
 * The bits combine.  Any other bit, or a bit with a bf16 cache, returns
 * ATTN_E_UNSUPPORTED.  Layout, limits and errors otherwise as
 * attn_paged_prefill; query elements must be finite.
 */
int attn_paged_prefill_fp8(const void* q, int32_t n_rows, const void* k_pool,
                           const void* v_pool, const float* k_scale, const float* v_scale,
                           int64_t n_pages, const int32_t* block_table,
                           int32_t max_pages_per_seq, int32_t ctx_len, int32_t n_head,
                           int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                           attn_kv_dtype kv_dtype, int32_t prefill_fp8, void* out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_paged_mixed -- a continuous-batching step: decode rows of
 * n_seq_decode sequences beside prefill chunks of the other sequences, in
 * one call ("Radiance Architecture Plugins -- declaring a model", section
 * "Step: issuing the graph": the core orders a mixed step decode-first, the
 * decode path runs over the first n_seq_decode sequences and the chunked
 * path over the rest, whose token offsets in cu_seqlens are absolute).
 *
 *   q, out       bf16 [n_tok][n_head][head_dim], token rows in step order
 *   cu_seqlens   int32 [n_seq + 1], DEVICE: sequence s owns token rows
 *                cu_seqlens[s] .. cu_seqlens[s + 1] - 1.  Decode-first:
 *                sequence s < n_seq_decode owns exactly row s.  Only the
 *                entries from n_seq_decode on are read (NULL allowed when
 *                n_seq_decode == n_seq).
 *   block_table  int32 [n_seq][max_pages_per_seq]
 *   ctx_lens     int32 [n_seq], DEVICE: lengths after this call
 *   max_q_len    HOST bound on the rows of any chunk (sizes the grid); the
 *                chunks' own row counts stay on the device
 *   workspace    attn_paged_workspace_bytes(3, n_seq_decode, ...)
 * Each decode row is bit for bit what attn_paged_decode returns for its
 * sequence, and each chunk row what attn_paged_prefill returns for its
 * chunk (the same per-row arithmetic).  With both halves present the chunk
 * half runs on a second stream the library keeps per device (made on first
 * use, default priority, kept until the process ends), forked from `stream`
 * and joined back to it by events inside the call, so to the caller all of
 * the call's work stays ordered on `stream`; the decode half then takes
 * seven eighths of the compute units.  Calls that overlap on one device
 * share that second stream and run their chunk halves in turn.  Host
 * checks: n_tok >= 1, 0 <= n_seq_decode <= n_seq, a chunk half needs
 * cu_seqlens, 1 <= max_q_len <= n_tok - n_seq_decode, and a decode-only step
 * has n_tok == n_seq.  On the device, a chunk whose rows fall outside
 * 1 .. max_q_len or past n_tok, or whose ctx_len is below its rows or
 * beyond the block-table row, is skipped (its rows of out are not written);
 * decode sequences follow the rules of attn_paged_decode.
 */
int attn_paged_mixed(const void* q, int32_t n_tok, const int32_t* cu_seqlens, int32_t n_seq,
                     int32_t n_seq_decode, int32_t max_q_len, const void* k_pool,
                     const void* v_pool, const float* k_scale, const float* v_scale,
                     int64_t n_pages, const int32_t* block_table, int32_t max_pages_per_seq,
                     const int32_t* ctx_lens, int32_t n_head, int32_t n_head_kv,
                     int32_t head_dim, int32_t page_size, attn_kv_dtype kv_dtype, void* out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Windowed and ring KV groups ("Radiance Architecture Plugins -- declaring a
 * model", section "Declare: buffers and KV groups": a KV group bounded by a
 * window, and a ring whose window floor is set at runtime).  A row at
 * position p attends keys lo .. p with
 *     lo = max(kv_floor, p - window + 1)      (window 0: no window)
 * Pages wholly below the first key a call's rows attend are neither read
 * nor checked, so a ring may have released them (their block-table entries
 * may hold anything).  A row's result depends only on its own position,
 * window and floor: every row of attn_paged_decode_window with `rows` rows
 * equals, bit for bit, the 1-row call at its position with the same window
 * and floor, and window 0 with floor 0 is the plain call.
 *
 * attn_paged_decode_window -- decode (rows = 1) or a round of rows <= 8,
 * layout and limits as attn_paged_verify_width.
 *   kv_floor  int32 [n_seq], DEVICE, or NULL (floor 0).  A floor outside
 *             0 .. ctx_lens[s] - rows gives NaN in every element of the
 *             sequence's rows.
 *   window    HOST value >= 0.
 */
int attn_paged_decode_window(const void* q, int32_t rows, const void* k_pool,
                             const void* v_pool, const float* k_scale, const float* v_scale,
                             int64_t n_pages, const int32_t* block_table,
                             int32_t max_pages_per_seq, const int32_t* ctx_lens, int32_t n_seq,
                             int32_t window, const int32_t* kv_floor, int32_t n_head,
                             int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                             attn_kv_dtype kv_dtype, void* out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * attn_paged_prefill_window -- attn_paged_prefill with the window and floor
 * above; window and kv_floor are HOST values, checked: window >= 0 and
 * 0 <= kv_floor <= ctx_len - n_rows.
 */
int attn_paged_prefill_window(const void* q, int32_t n_rows, const void* k_pool,
                              const void* v_pool, const float* k_scale, const float* v_scale,
                              int64_t n_pages, const int32_t* block_table,
                              int32_t max_pages_per_seq, int32_t ctx_len, int32_t window,
                              int32_t kv_floor, int32_t n_head, int32_t n_head_kv,
                              int32_t head_dim, int32_t page_size, attn_kv_dtype kv_dtype,
                              void* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * attn_kv_append -- write n_tok new K/V rows into their token slots
 * ("kern manifest v7" schema, $defs.Fill "slot": each row's token slot in
 * the paged state; slot = page * page_size + offset).  A negative slot skips
 * its row (bucket padding).
 *
 *   k_new, v_new  bf16 [n_tok][n_head_kv][head_dim]
 *   slot_mapping  int32 [n_tok]
 * bf16 pools: a copy.  fp8 pools: a page's K scale and V scale are set to
 * absmax / 448 (1 when absmax is 0) over this call's rows in that page, by
 * the call that writes the page's offset 0.  A call that writes only later
 * offsets keeps the stored scale s while its rows fit (fp32 absmax / s <=
 * 448); otherwise the scale doubles until they do, and the codes already in
 * the page's slots below the call's first one are re-encoded at the new
 * scale s' (nearest E4M3 to fp32(fp32(value * s) / s'), exact for codes that
 * stay normal), so a page filled one token per call keeps E4M3's precision.
 * Each new code is the E4M3 value nearest to the fp32 quotient x / scale,
 * ties to even, saturating at +-448.
 * Precondition for fp8: the rows a call writes into one page are adjacent
 * in the call, in increasing offset order (true of any sequence's run of
 * new tokens); two runs of one page in one call race on its scale.  Slots must lie below n_pages * page_size; a larger slot
 * skips its row.
 */
int attn_kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping,
                   int32_t n_tok, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                   int64_t n_pages, int32_t n_head_kv, int32_t head_dim, int32_t page_size,
                   attn_kv_dtype kv_dtype, hipStream_t stream);

/*
 * attn_block_table_build -- HOST helper that deals each sequence its own
 * pages from a pool of pool_pages pages.
 *
 * The pool's page ids are shuffled by a Fisher-Yates (Durstenfeld) pass
 * driven by Vigna's splitmix64 seeded with `seed` (swap partner of position
 * i = next() mod (i + 1), i from pool_pages-1 down to 1); sequence s, in
 * order, then takes the next ceil(ctx_lens_host[s] / page_size) ids.
 * Unused columns are -1.  If slot_mapping_host is not NULL it receives, for
 * every sequence in order and every position t < ctx_lens_host[s], the slot
 * block_table[s][t / page_size] * page_size + t % page_size.
 * Returns ATTN_E_RANGE when a context needs more than max_pages_per_seq
 * pages or the pool is too small.
 */
int attn_block_table_build(int32_t n_seq, const int32_t* ctx_lens_host, int32_t page_size,
                           int64_t pool_pages, uint64_t seed, int32_t max_pages_per_seq,
                           int32_t* block_table_host, int32_t* slot_mapping_host);

/* op: 0 decode, 1 verify, 2 prefill, 3 mixed (n_seq = the step's
   n_seq_decode), 4 tree round (any width).  Bytes of device workspace the call needs; 0 for an
   unsupported combination. */
size_t attn_paged_workspace_bytes(int op, int32_t n_seq, int32_t max_pages_per_seq,
                                  int32_t n_head, int32_t head_dim);

/* ATTN_OK if the kernels serve this (head_dim, page_size, kv_dtype),
   else ATTN_E_UNSUPPORTED (the counterpart of the pages' probe bits). */
int attn_caps(int32_t head_dim, int32_t page_size, attn_kv_dtype kv_dtype);

/* HOST checks of device-resident inputs, for callers holding host copies.
   attn_check_lengths_host: rows <= ctx_lens[s] <= max_pages*page_size.
   attn_check_block_table_host: every entry a sequence reads is in
   [0, n_pages).  Return ATTN_OK or ATTN_E_RANGE (message names s). */
int attn_check_lengths_host(const int32_t* ctx_lens_host, int32_t n_seq, int32_t rows,
                            int32_t max_pages_per_seq, int32_t page_size);
int attn_check_block_table_host(const int32_t* block_table_host, const int32_t* ctx_lens_host,
                                int32_t n_seq, int32_t max_pages_per_seq, int32_t page_size,
                                int64_t n_pages);

/*
 * attn_check_device -- checked mode on the device, for callers without host
 * copies ("kern manifest v7" schema, $defs.Domain: out-of-domain inputs are
 * rejected; $defs.Fill "error": a one-word error flag read after the call).
 * Enqueues a check of what a call with these arguments would read: every
 * ctx_lens[s] in rows .. max_pages_per_seq * page_size, and every block-table
 * entry of a page holding a key some row attends (pages wholly below the
 * first key of the first row -- window and kv_floor as for
 * attn_paged_decode_window, 0 / NULL for none -- are skipped) in
 * [0, n_pages).  *err_word (device int64) becomes -1 when all hold, else
 * s * (max_pages_per_seq + 1) + e + 1 for the first failure in (sequence,
 * entry) order, e = -1 naming the length.  Read it after the stream has
 * passed the call.
 */
int attn_check_device(const int32_t* block_table, const int32_t* ctx_lens,
                      const int32_t* kv_floor, int32_t window, int32_t n_seq, int32_t rows,
                      int32_t max_pages_per_seq, int32_t page_size, int64_t n_pages,
                      int64_t* err_word, hipStream_t stream);

/* Message of the last failing call on this thread ("" after a success). */
const char* attn_last_error(void);

/*
 * Measurement hook: the next decode, verify or prefill call made on this
 * thread records `start` just before and `stop` just after its main
 * attention kernel (a mixed call: around both of its halves), on the call's
 * stream, then forgets both.  Pass NULLs to
 * cancel.  Lets a benchmark time that kernel alone with HIP events.
 */
void attn_set_kernel_timer(hipEvent_t start, hipEvent_t stop);

/*
 * Upper bound on the workgroups of the decode / verify attention kernel for
 * every later call in the process (0, the default, lets the grid fill the
 * device; negative values count as 0).  The kernel's waves walk the work
 * items whatever their number, and results do not depend on it, so a small
 * bound lets tests drive many work items through each wave on small inputs.
 */
void attn_set_max_workgroups(int32_t n);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDATTN_H */
