/*
 * ftm.h -- C ABI of libftm: fused decode-step masked multi-head attention
 * over a KV cache, for AMD Instinct MI355X (gfx950).
 *
 * One call performs one decode step of one attention layer for a batch of
 * sequences.  For every sequence b and every query head h it
 *   1. adds the QKV bias to the step's query and to its new key/value row
 *      ([lpnh.cn/news/2765398] section 2.1: Q, K and V come out of one fused
 *      projection, are split three ways and carry their bias);
 *   2. appends the biased new K/V row to a pre-allocated cache
 *      ([lpnh.cn/news/2765398] section 2.2; [intelliparadigm.com .../2131745]
 *      section 2.1: the cache is allocated once and filled position by
 *      position; [framerc.cn/news/4453289] section 3.2);
 *   3. dots the single query with every cached key, scaled by 1/sqrt(D);
 *   4. takes a softmax with the maximum subtracted
 *      ([lpnh.cn/news/2765398] section 6.1: Q.K can leave the fp16 range
 *      without care; [intelliparadigm.com .../2131745] section 6.2);
 *   5. forms the softmax-weighted sum of the cached values,
 * in fused kernels that never write a score matrix to memory
 * ([lpnh.cn/news/2765398] section 2.1; [framerc.cn/news/4453289] section 2.2).
 *
 * All pointers are caller-owned device pointers unless stated otherwise.
 * Errors are returned before anything is enqueued; the library never aborts
 * the process (FasterTransformer aborts on a bad length,
 * [lmnt.cn/news/219530] section 5.2).
 *
 * Blocking.  The compute calls (ftm_decode_mha, ftm_decode_mha_paged,
 * ftm_decode_mha_static, ftm_qkv_proj, ftm_prefill_mha,
 * ftm_prefill_mha_paged) only enqueue work on their stream and return: they
 * never wait for the device and never read device memory on the host
 * (there is no synchronisation on the decode path,
 * [lmnt.cn/news/219530] section 6.1).  A call that needs a larger
 * workspace allocates it with hipMalloc and clears what must start at zero
 * with a kernel on the call's stream; the buffer it replaces is kept, not
 * freed (hipFree would wait for the device), until
 * ftm_release_workspaces.  The calls that do wait: ftm_release_workspaces
 * (frees), ftm_timing_read (waits for the events it reads), and any compute
 * call while FTM_VALIDATE=1 is set in the environment (it copies seq_lens to
 * the host and waits for the stream).  ftm_graph_end and ftm_graph_destroy
 * instantiate and free graphs on the host and may wait for the device.
 */
#ifndef FTM_H
#define FTM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle, as hip_runtime_api.h declares it (a repeated
 * identical typedef is valid C11 and C++).  NULL is the null stream. */
typedef struct ihipStream_t* hipStream_t;

/* Cache element types ([lpnh.cn/news/2765398] section 6.1 and
 * [intelliparadigm.com .../2131745] section 4.1: fp16/bf16 storage;
 * [pptc.cn/news/144085] section 3.1: an INT8 KV cache). */
typedef enum {
    FTM_F32 = 0,
    FTM_F16 = 1,
    FTM_BF16 = 2,
    FTM_I8 = 3
} ftm_dtype;

typedef enum {
    FTM_OK = 0,
    FTM_ERR_INVALID_ARG = 1,   /* null pointer, bad size, inconsistent shapes   */
    FTM_ERR_UNSUPPORTED = 2,   /* valid but not built: head_dim, head grouping  */
    FTM_ERR_HIP = 3,           /* a HIP runtime call or kernel launch failed    */
    FTM_ERR_OUT_OF_MEMORY = 4  /* the library's split workspace could not grow  */
} ftm_status;

/*
 * ftm_decode_mha -- one decode step of masked multi-head attention.
 *
 * Shapes (row-major, contiguous, D = head_dim, G = n_heads / n_kv_heads):
 *   q         [batch, n_heads, D]             act type, read
 *   k_new     [batch, n_kv_heads, D]          act type, read
 *   v_new     [batch, n_kv_heads, D]          act type, read
 *   qkv_bias  [(n_heads + 2 n_kv_heads) D]    act type, read; [b_q | b_k | b_v],
 *             each head-major, shared by all sequences; NULL means no bias
 *   k_cache, v_cache [batch, n_kv_heads, max_seq_len, D]  kv_dtype, read, and
 *             row seq_lens[b]-1 of every (b, KV head) written
 *   seq_lens  [batch] int32 device array, or NULL (every length = step).
 *             seq_lens[b] counts the token appended by this call: the new
 *             row goes to position seq_lens[b]-1 and the query attends to
 *             positions [0, seq_lens[b]).
 *   step      the largest seq_lens[b]; 1 <= step <= max_seq_len
 *   kv_scales [2, batch, n_kv_heads, max_seq_len] fp32, INT8 caches only
 *             (K scales first, then V): read at positions below the new
 *             row, written at the new row; must be NULL otherwise
 *   out       [batch, n_heads, D]             act type, written
 *   stream    a hipStream_t; NULL is the null stream
 * The act type is kv_dtype for float caches and fp16 for an INT8 cache.
 *
 * Arithmetic: the bias add is an fp32 add; the appended row is stored
 * rounded to nearest even (fp16/bf16), as is (fp32), or as symmetric INT8
 * codes rint(x / s) clamped to [-127, 127] with s = absmax(row) / 127 (a
 * zero row stores s = 0 and zero codes).  The attention reads the stored
 * values back (INT8: code * scale), accumulates in fp32 and writes out
 * rounded to nearest even.  Query head h uses KV head h / G
 * ([pptc.cn/news/144085] section 3.4: heads share K/V in groups).
 *
 * Supported: head_dim 64 or 128; any n_heads that is a multiple of
 * n_kv_heads.  Up to 8 query heads of a group are served by one pass over
 * the group's K/V; larger groups take one pass per 8 heads.
 *
 * Alignment: q, k_new, v_new, qkv_bias, k_cache, v_cache and out 16 bytes
 * (every row of D elements then starts on a 16-byte boundary); seq_lens and
 * kv_scales 4 bytes.
 *
 * Errors (nothing is enqueued): FTM_ERR_INVALID_ARG for a null required
 * pointer, a misaligned pointer, non-positive sizes, n_heads % n_kv_heads != 0, step outside
 * [1, max_seq_len], an unknown kv_dtype, or kv_scales given/missing against
 * the cache type; FTM_ERR_UNSUPPORTED for another head_dim;
 * FTM_ERR_OUT_OF_MEMORY if the internal workspace cannot grow;
 * FTM_ERR_HIP if a launch fails.  ftm_last_error() tells which.
 * A sequence whose device-side length lies outside [1, step] is not
 * appended and gets NaN output rows (no host synchronisation is needed to
 * see the error).
 *
 * Ownership: the library never frees or keeps caller pointers.  It owns one
 * split-sequence workspace per (device, stream), grown on the first call
 * that needs more and reused afterwards.  out must not alias any input.
 * Calls on different streams may run concurrently; calls that share a cache
 * row on different streams race, as any two writers would.
 */
int ftm_decode_mha(const void* q, const void* k_new, const void* v_new,
                   const void* qkv_bias, void* k_cache, void* v_cache,
                   const int32_t* seq_lens, int batch, int max_seq_len, int step,
                   int n_heads, int n_kv_heads, int head_dim, ftm_dtype kv_dtype,
                   float* kv_scales, void* out, hipStream_t stream);

/*
 * ftm_decode_mha_static -- ftm_decode_mha without any allocation.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, kernels, results and errors as ftm_decode_mha, but the
 * scratch memory of the step (the split partials and the per-unit counters
 * of the grouped-query pass) is a fixed device array of 8 MiB that each GPU
 * holds from the library's first use until the process ends, instead of
 * the per-stream workspace.  The call never calls hipMalloc or hipFree; the
 * first call on a device that needs scratch takes the array's address
 * (hipGetSymbolAddress) and clears its counters with a kernel on `stream`.
 *
 * Limit: a step whose scratch exceeds the array returns FTM_ERR_UNSUPPORTED
 * before anything is enqueued: at most 8 MiB - 64 KiB of partials
 * (batch * n_heads * chunks * (head_dim + 2) * 4 bytes for a split pass;
 * 2 * workgroups * group tile * (head_dim + 2) * 4 for the grouped-query
 * pass) and 16384 (sequence, KV head, head group) units.  A single pass
 * needs no scratch.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (on different streams, or on different host threads)
 * race and give wrong results.  Serialise them, or use ftm_decode_mha,
 * whose workspace is per stream.
 */
int ftm_decode_mha_static(const void* q, const void* k_new, const void* v_new,
                          const void* qkv_bias, void* k_cache, void* v_cache,
                          const int32_t* seq_lens, int batch, int max_seq_len, int step,
                          int n_heads, int n_kv_heads, int head_dim, ftm_dtype kv_dtype,
                          float* kv_scales, void* out, hipStream_t stream);

/*
 * ftm_decode_mha_paged -- the same decode step over a paged KV cache.
 *
 * The cache is cut into fixed-size pages that sequences take as needed,
 * as in virtual memory ([intelliparadigm.com .../2131745] section 5.1: a
 * cache split into pages of a fixed number of tokens; [framerc.cn/news/
 * 4453289] section 3.2: fixed-size blocks allocated on demand instead of
 * one maximum-length buffer per sequence).  Position i of sequence b lives
 * in page block_table[b][i / page_size], at row i % page_size.
 *
 * Shapes (row-major, contiguous; P = page_size):
 *   k_pages, v_pages [n_pages, n_kv_heads, P, D]  kv_dtype, read, and the
 *             row of position seq_lens[b]-1 of every (b, KV head) written
 *   block_table [batch, max_pages_per_seq] int32 device array: page indices
 *             in [0, n_pages); only the entries of pages holding positions
 *             below seq_lens[b] are read
 *   kv_scales [2, n_pages, n_kv_heads, P] fp32, INT8 caches only (K scales
 *             first), read and written like the rows they scale
 *   every other argument as for ftm_decode_mha, with max_pages_per_seq * P
 *             in the role of max_seq_len (step <= max_pages_per_seq * P).
 * Arithmetic, the append rule and the results are those of ftm_decode_mha
 * on the cache the table describes.  page_size must be a power of two in
 * [16, 65536]; k_pages and v_pages 16-byte aligned, block_table 4 bytes.
 *
 * The caller owns the pool and the table.  Pages that two sequences share,
 * or that one sequence lists twice, are the caller's to keep consistent:
 * the call writes one row per (sequence, KV head) and reads the others
 * concurrently.  A sequence whose table names a page outside [0, n_pages)
 * at a position it reads gets NaN output rows; when that page is the one
 * of the new row, the row is not appended (no host synchronisation is
 * needed to see the error).  Other errors as for ftm_decode_mha, plus
 * FTM_ERR_INVALID_ARG for a NULL or misaligned block_table, n_pages or
 * max_pages_per_seq below 1, or another page_size.
 * ftm_kv_cache_bytes(n_pages, n_kv_heads, page_size, head_dim, kv_dtype)
 * gives the pool's bytes.
 */
int ftm_decode_mha_paged(const void* q, const void* k_new, const void* v_new,
                         const void* qkv_bias, void* k_pages, void* v_pages,
                         const int32_t* block_table, int n_pages, int page_size,
                         int max_pages_per_seq, const int32_t* seq_lens, int batch, int step,
                         int n_heads, int n_kv_heads, int head_dim, ftm_dtype kv_dtype,
                         float* kv_scales, void* out, hipStream_t stream);

/*
 * ftm_qkv_proj -- the fused QKV projection that feeds a decode step.
 *
 * One projection produces Q, K and V for every sequence and its output is
 * split three ways straight into the layouts ftm_decode_mha reads
 * ([lpnh.cn/news/2765398] section 2.1: Q, K and V from one fused kernel,
 * split without an extra write; section 1.2: every decode step reads the
 * whole weight matrix):
 *   y = x W^T (+ bias),  q = y[:, 0 : H D],  k_new = y[:, H D : (H + Hkv) D],
 *   v_new = y[:, (H + Hkv) D :], each reshaped per head.
 *
 * Shapes (row-major, contiguous; N = (n_heads + 2 n_kv_heads) head_dim):
 *   x      [batch, hidden]     act_dtype, read
 *   w      [N, hidden]         act_dtype, read (one row of weights per output feature)
 *   bias   [N] act_dtype or NULL
 *   q      [batch, n_heads, head_dim]      act_dtype, written
 *   k_new, v_new [batch, n_kv_heads, head_dim]  act_dtype, written
 * act_dtype is FTM_F16 or FTM_BF16.  Products accumulate in fp32 (on the
 * matrix cores), the bias is added in fp32, and the result is rounded to
 * nearest even.  When the bias is added here, pass qkv_bias = NULL to
 * ftm_decode_mha (or add it there instead, and pass NULL here).
 *
 * Batches above 32 rows may split the hidden dimension over two to four
 * workgroups per 128 output features; their fp32 partial sums then go
 * through the stream's workspace (batch rounded up to 16, times 512 bytes
 * per workgroup, at most about 8 MiB on 256 CUs) and are added in a fixed
 * order, so the result does not depend on timing.  Under stream capture
 * that workspace must already exist: make one eager call of the shape on
 * the stream first.
 *
 * Supported: batch 1..64, hidden a multiple of 256 up to 65536, head_dim a
 * multiple of 16.  All pointers 16-byte aligned; q, k_new and v_new must
 * not overlap x or w.  Errors as for ftm_decode_mha (FTM_ERR_UNSUPPORTED for
 * fp32 or sizes outside the supported set, FTM_ERR_OUT_OF_MEMORY if the
 * workspace cannot grow).  Only enqueues on `stream`.
 */
int ftm_qkv_proj(const void* x, const void* w, const void* bias, void* q, void* k_new,
                 void* v_new, int batch, int hidden, int n_heads, int n_kv_heads, int head_dim,
                 ftm_dtype act_dtype, hipStream_t stream);

/*
 * ftm_prefill_mha -- prefill: the whole prompt of every sequence in one step.
 *
 * The prompt is processed in parallel where decode goes token by token
 * ([lpnh.cn/news/2765398] section 1.1): the prompt's K/V rows (bias added
 * in fp32, rounded to nearest even) are written to cache positions
 * [0, S_b), and every prompt position t of every query head attends
 * causally to positions [0, t] of its KV head, reading the stored rows.
 * Position t gets what ftm_decode_mha computes at length t + 1, with the
 * same readings (scale 1/sqrt(D), maximum subtracted, fp32 accumulation).
 *
 * Shapes (row-major, contiguous; S = prompt_len):
 *   q         [batch, S, n_heads, D]      read
 *   k_new, v_new [batch, S, n_kv_heads, D]  read
 *   qkv_bias  [(n_heads + 2 n_kv_heads) D] or NULL
 *   k_cache, v_cache [batch, n_kv_heads, max_seq_len, D]  rows [0, S_b) written
 *   seq_lens  [batch] int32 prompt lengths S_b in [1, S], or NULL (all S)
 *   out       [batch, S, n_heads, D]      rows t < S_b written, the rest untouched
 * kv_dtype FTM_F16 or FTM_BF16 (activations of the same type) or FTM_I8
 * (fp16 activations); head_dim 64 or 128; S <= max_seq_len.  A sequence
 * whose length lies outside [1, S] is not appended and gets NaN rows.
 *
 * INT8 cache: kv_scales [2, batch, n_kv_heads, max_seq_len] fp32 (K first),
 * NULL otherwise.  Each prompt row is quantised as a decode step quantises
 * its new row (s = absmax / 127, code = round-to-nearest-even of x / s
 * clamped to [-127, 127]) and the attention uses code x scale, as decode
 * does.  The library then stages the prompt's codes (as fp16) and scales
 * in its per-stream workspace (4 batch n_kv_heads S (head_dim + 2) bytes),
 * allocated on the first call of a larger shape; under stream capture a
 * call that would grow it is refused, as for ftm_decode_mha.  The attention
 * multiplies each raw score by its key's K scale and each softmax weight
 * (at most 2^8 against the running reference) by its key's V scale in
 * fp32 before the weight enters the matrix cores in fp16; the staging
 * holds V codes times 8 and V scales divided by 8, so that product stays
 * within the fp16 range for every finite fp16 input and bias (only a power
 * of two moves between the two factors).  INT8 limits: prompt_len * head_dim * 2 and
 * prompt_len * n_kv_heads * head_dim / 16 below 2^31 (FTM_ERR_UNSUPPORTED).
 * Two kernels are enqueued (append, then attention).  The attention runs on
 * the matrix cores with fp32
 * accumulation: the query enters exactly as stored and the bias term
 * b_q . k separately (once per key and head), so the scores are exact
 * products summed in fp32 and then scaled.  Over fp16/bf16 caches with a
 * bias the append computes those terms into the stream's workspace
 * (4 batch n_heads S bytes), grown on the first call of a larger shape as
 * for the INT8 staging (so a capture needs one eager call of the shape on
 * the stream first).  fp16 softmax weights are
 * rounded once to nearest (11 significant bits); bf16 weights, and those
 * over INT8 codes, enter as hi and lo halves, so about 16 (bf16) or 22
 * (fp16) bits of each reach the accumulators.  Limits: batch up to 65535,
 * batch * n_heads below 2^31, prompt_len up to 65535 * 128.  Errors as for
 * ftm_decode_mha.
 */
int ftm_prefill_mha(const void* q, const void* k_new, const void* v_new, const void* qkv_bias,
                    void* k_cache, void* v_cache, const int32_t* seq_lens, int batch,
                    int max_seq_len, int prompt_len, int n_heads, int n_kv_heads, int head_dim,
                    ftm_dtype kv_dtype, float* kv_scales, void* out, hipStream_t stream);

/*
 * ftm_prefill_mha_paged -- prefill into a paged KV cache.
 *
 * The same prefill as ftm_prefill_mha, with the cache cut into fixed-size
 * pages located through a block table ([intelliparadigm.com
 * /article/weixin_32285357/2131745] section 5.1; [framerc.cn/news/4453289]
 * section 3.2): position t of sequence b is row t mod P of page
 * block_table[b, t / P], in the layout ftm_decode_mha_paged reads.
 *
 *   k_pages, v_pages [n_pages, n_kv_heads, page_size, D]  rows of the
 *                     prompt positions written, every other row untouched
 *   block_table [batch, max_pages_per_seq] int32, device; only the entries
 *                     of pages holding positions < S_b are read
 * page_size is a power of two in [16, 65536]; prompt_len <= max_pages_per_seq
 * * page_size.  A table entry outside [0, n_pages) among the pages of
 * positions [0, S_b) makes the sequence's output rows [0, S_b) NaN, and no
 * row is appended into such a page (the rows of its valid pages are).
 * INT8: kv_scales [2, n_pages, n_kv_heads, page_size] fp32 (K first), the
 * scales of the pooled rows, in the layout ftm_decode_mha_paged reads.
 * Everything else (shapes of q, k_new, v_new, qkv_bias, seq_lens, out,
 * numerics, limits, errors, the two kernels) is ftm_prefill_mha's.
 */
int ftm_prefill_mha_paged(const void* q, const void* k_new, const void* v_new, const void* qkv_bias,
                          void* k_pages, void* v_pages, const int32_t* block_table, int n_pages,
                          int page_size, int max_pages_per_seq, const int32_t* seq_lens, int batch,
                          int prompt_len, int n_heads, int n_kv_heads, int head_dim, ftm_dtype kv_dtype,
                          float* kv_scales, void* out, hipStream_t stream);

/* ---- HIP graphs ----------------------------------------------------------
 * A decode step of a model is one call per layer on fixed buffers; its
 * kernel launches can be recorded once and replayed as one graph launch, so
 * that launch overhead stops dominating small shapes ([lmnt.cn/news/219530]
 * section 5.3 and [lpnh.cn/news/2765398] section 1.2: the count of kernel
 * launches per decode step is a cost of its own; [pptc.cn/news/144085]
 * section 2.3).
 *
 * ftm_graph_begin starts capturing `stream` (a created stream, not the null
 * stream; capture mode thread-local).  The ftm_decode_mha, ftm_decode_mha_paged,
 * ftm_qkv_proj, ftm_prefill_mha and ftm_prefill_mha_paged calls that follow
 * on that stream and host thread are recorded, not run.  They allocate nothing: each needs a workspace that an
 * earlier call of the same or a larger shape on the same stream has already
 * grown, or it fails with FTM_ERR_INVALID_ARG and records nothing (the
 * capture stays valid).  FTM_VALIDATE and kernel timing do not apply while
 * capturing.  ftm_graph_end stops the capture and instantiates the graph
 * into *graph (NULL on failure).  ftm_graph_launch replays it on any stream:
 * the same kernels on the same pointers, reading the buffers' contents at
 * replay time.  Replays of one graph, and calls on the stream it was
 * captured on, share that stream's workspace: do not run them concurrently.
 * A workspace a graph was captured with stays allocated when a later call
 * needs a larger one, so graphs stay valid until ftm_release_workspaces,
 * after which they must not be replayed.
 * ftm_graph_destroy frees the graph (NULL is accepted).  All return FTM_OK
 * or FTM_ERR_INVALID_ARG / FTM_ERR_HIP with ftm_last_error() set.
 */
typedef struct ftm_graph_s* ftm_graph;
int ftm_graph_begin(hipStream_t stream);
int ftm_graph_end(hipStream_t stream, ftm_graph* graph);
int ftm_graph_launch(ftm_graph graph, hipStream_t stream);
int ftm_graph_destroy(ftm_graph graph);

/* Bytes of one layer's K and V cache (plus INT8 scales) for the layout
 * above: 2 * batch * n_kv_heads * max_seq_len * (head_dim * elem + scale),
 * scale = 4 bytes for INT8, 0 otherwise.  Sizing as in
 * [pptc.cn/news/144085] section 3.1 (batch x length x layers x hidden x
 * bytes, counted for K and V).  Returns 0 for invalid arguments. */
size_t ftm_kv_cache_bytes(int batch, int n_kv_heads, int max_seq_len, int head_dim,
                          ftm_dtype kv_dtype);

/* Message for the last failed call on this host thread ("" if none).
 * Owned by the library; valid until the next call on this thread.  Errors
 * are returned as a status with this message instead of aborting the
 * process, which is what FasterTransformer does when a length passes the
 * cache's capacity ([lmnt.cn/news/219530] section 5.2). */
const char* ftm_last_error(void);

/* Library version string ("libftm <version> (gfx950)"), owned by the
 * library.  Not a step of the method: it names the build a caller loaded. */
const char* ftm_version(void);

/* Chunk length, in positions, of the split-sequence pass (flash-decoding:
 * independent partial softmax states per chunk, merged by a combine
 * kernel; [pptc.cn/news/144085] section 2.2 on running softmax statistics).
 * 0 restores the automatic choice.  Values are rounded up to the kernel's
 * tile; a chunk of `step` or more gives a single pass with no combine.
 * Process-wide; returns the previous setting, or -1 for a negative value. */
int ftm_set_split_chunk(int positions);

/* Waves per workgroup of the attention pass: 4 or 16; 0 restores the
 * automatic choice (16 when there are fewer (sequence, KV head) units than
 * twice the CU count and the 16-wave shape is built, else 4).  The 16-wave
 * shape is built for passes of one query head over fp32, fp16 and bf16
 * caches; elsewhere 4 is used whatever is set.  Process-wide; returns the
 * previous setting, or -1 for another value. */
int ftm_set_workgroup_waves(int waves);

/* Frees every workspace the library holds (all devices and streams),
 * including the buffers that larger ones replaced.  Workspaces are
 * allocated once and reused across calls and layers instead of per call
 * ([lpnh.cn/news/2765398] section 2.2: intermediate buffers are pooled
 * and recycled; [lmnt.cn/news/219530] section 6.4), so this is the one
 * place they are freed.  It waits for the device (hipFree).  The caller
 * must make sure no call of this library is still running, and must not
 * replay graphs captured before the release. */
void ftm_release_workspaces(void);

/* Re-reads the tuning variables of the environment (FTM_VALIDATE,
 * FTM_WAVES, FTM_SPLIT_CHUNK, FTM_GQA_VALU, FTM_GQA_BLOCKS_PER_CU,
 * FTM_GQA_UNIT_COST, FTM_GQA_SKEW, FTM_QKV_COLUMN_TILES, FTM_QKV_K_SPLIT).  The library
 * reads them once, at its first call, and not again on the call path;
 * a process that changes them calls this afterwards.  Not a step of the
 * method: the variables choose launch shapes for measurement and tests. */
void ftm_tuning_reload(void);

/* ---- kernel timing -------------------------------------------------------
 * For measurement only.  While enabled, every ftm_decode_mha(_paged) and
 * ftm_prefill_mha(_paged) call records a HIP event pair around each kernel it
 * launches, on the call's stream (not while the stream is being captured).
 * ftm_timing_read() waits for the recorded events, returns the number of
 * launches and their summed duration in milliseconds for one kernel kind
 * and clears that kind's records.  Kinds: 0 = attention pass (decode: split
 * or single-pass; prefill: the causal attention), 1 = decode: combine,
 * prefill: the append of the prompt's K/V rows.  At most `capacity`
 * launches are kept per kind; later ones are not recorded.  Returns FTM_OK
 * or an error. */
int ftm_timing_enable(int capacity);
int ftm_timing_disable(void);
int ftm_timing_read(int kind, int* launches, double* total_ms);

#ifdef __cplusplus
}
#endif
#endif /* FTM_H */
