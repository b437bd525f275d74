/*
 * kvsel — query-aware sparse-page decode attention over a paged GQA KV cache, for AMD Instinct
 * MI355X (gfx950). C ABI of libkvsel.so.
 *
 * The operations follow these pages (cited by title and section):
 *  [FreeKV]   "FreeKV: Boosting KV Cache Retrieval for Efficient LLM Inference" (Korean summary),
 *             technical summary section 1 (keep the whole KV cache, use only the part a step
 *             needs) and section 2.1 (choose KV pages per KV head with the current query; reuse
 *             the previous step's pages; correct a KV head when its group-mean query similarity
 *             is below tau).
 *  [KV wiki]  "Key-Value (KV) Cache" wiki page: paged storage (PagedAttention entry), grouped-query
 *             heads (Graph entry), decode bound by memory bandwidth (bottleneck entry).
 *  [KV Packet] "[Paper review] KV Packet: Recomputation-Free Context-Independent KV Caching for
 *             LLMs", section 1: RoPE re-aligns precomputed KV states to new positions.
 * Where the pages leave a step open, the header states the rule this library implements.
 *
 * Conventions shared by every call
 *  - Shapes: B sequences, Hq query heads, Hkv KV heads (G = Hq / Hkv; query head h reads KV head
 *    h / G), head dim D in {64, 128}, page size P in {16, 32}, G in {1, 2, 4, 8}.
 *  - Element type (kvsel_paged_kv.dtype): KVSEL_F32 (float) or KVSEL_BF16 (bfloat16 bits in
 *    uint16). K, V, q, summaries and attention outputs all use it. KVSEL_FP8_E4M3: K and V
 *    pools hold 8-bit codes with one fp32 scale per (physical page, KV head) tile (k_scale,
 *    v_scale; see kvsel_quantize_pages); q, summaries and outputs are then bfloat16 ("the element
 *    type" below means bfloat16 for them). Calls on an fp8 cache take no rotary argument, and
 *    kvsel_append_kv and kvsel_rope_shift do not take an fp8 cache (KVSEL_ERR_UNSUPPORTED).
 *  - Pools: k_pool is [num_phys_pages][Hkv][P][D] (token-major pages: key of physical page p,
 *    KV head j, slot s starts at element ((p * Hkv + j) * P + s) * D). v_pool is
 *    [num_phys_pages][Hkv][D][P] (channel-major pages: channel d of the values of page p, head j
 *    is the run of P slots starting at ((p * Hkv + j) * D + d) * P), so that the probability x
 *    value contraction over a page's tokens reads consecutive tokens.
 *  - page_table is int32 [B][max_pages_per_seq]: logical page n of sequence b lives in physical
 *    page page_table[b][n]. seq_lens is int32 [B]; sequence b has N_b = ceil(seq_lens[b] / P)
 *    logical pages, and slot s of logical page n is valid iff n * P + s < seq_lens[b]. Table
 *    entries at or past N_b and invalid slots are never read (they may hold anything).
 *  - All pointers in the descriptors and arguments are DEVICE pointers unless marked host, and
 *    must stay valid until the work enqueued on `stream` completes. The caller owns every buffer;
 *    the library allocates, frees and retains no memory.
 *  - `stream` is a hipStream_t (NULL = the null stream). Every call only enqueues work and returns
 *    without synchronizing; outputs are ready when the stream reaches that point.
 *  - Errors: arguments are validated on the host BEFORE anything is enqueued, so a failing call
 *    has no effect. Device-side contents (page ids in range, seq_lens <= the live bound, i.e.
 *    max_seq_len if set, else max_pages_per_seq * P; selected ids < N_b) are the caller's
 *    contract and are not checked.
 */
#ifndef KVSEL_H
#define KVSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVSEL_ABI_VERSION 7

typedef int32_t kvsel_status;
#define KVSEL_OK 0
#define KVSEL_ERR_INVALID_ARGUMENT 1 /* NULL required pointer, size < 1, Hq % Hkv != 0, ...  */
#define KVSEL_ERR_UNSUPPORTED 2      /* D, P, G, dtype or size without a kernel               */
#define KVSEL_ERR_WORKSPACE 3        /* workspace NULL or smaller than kvsel_workspace_bytes */
#define KVSEL_ERR_DEVICE 4           /* current device is not gfx950, or no device           */
#define KVSEL_ERR_LAUNCH 5           /* the HIP runtime rejected a launch                    */
#define KVSEL_ERR_SCRATCH 6          /* the call needs more than KVSEL_STATIC_SCRATCH_BYTES    */

/* Size of the library's device-resident scratch array (kvsel_select_attend_static). */
#define KVSEL_STATIC_SCRATCH_BYTES (8u << 20)

/* Largest supported batch and page-table width (launch-grid limits). */
#define KVSEL_MAX_BATCH 65535
#define KVSEL_MAX_PAGES_PER_SEQ 1048576

#define KVSEL_F32 0
#define KVSEL_BF16 1
#define KVSEL_FP8_E4M3 2 /* pools only: OCP FP8 E4M3 codes + per-tile fp32 scales */

/* Workspace kinds for kvsel_workspace_bytes. */
#define KVSEL_OP_SCORE_TOPK 1
#define KVSEL_OP_ATTENTION 2
#define KVSEL_OP_SELECT_ATTEND 3
#define KVSEL_OP_SPECULATIVE_STEP 4

/* Flags of kvsel_score_topk. */
#define KVSEL_SCORE_REFRESH_TAIL 1 /* rebuild each sequence's last-page summary first */

/* Host struct describing one paged KV cache (device pointers inside). */
typedef struct kvsel_paged_kv {
  int32_t dtype;             /* KVSEL_F32, KVSEL_BF16 or KVSEL_FP8_E4M3               */
  int32_t batch;             /* B                                                    */
  int32_t num_q_heads;       /* Hq                                                   */
  int32_t num_kv_heads;      /* Hkv                                                  */
  int32_t head_dim;          /* D                                                    */
  int32_t page_size;         /* P                                                    */
  int32_t num_phys_pages;    /* pages in the pool                                    */
  int32_t max_pages_per_seq; /* row length of page_table                             */
  const void* k_pool;        /* [num_phys_pages][Hkv][P][D]                          */
  const void* v_pool;        /* [num_phys_pages][Hkv][D][P] (may be NULL where unused) */
  const int32_t* page_table; /* [B][max_pages_per_seq]                               */
  const int32_t* seq_lens;   /* [B]                                                  */
  int32_t max_seq_len;       /* 0, or the caller's bound on every seq_lens[b] (host)  */
  const float* k_scale;      /* fp8 only: [num_phys_pages][Hkv] fp32 (else ignored)   */
  const float* v_scale;      /* fp8 only: [num_phys_pages][Hkv] fp32, with v_pool     */
  const int32_t* page_fill;  /* [num_phys_pages] valid slots per page (1..P), or NULL  */
} kvsel_paged_kv;

/* page_fill: a sequence may chain pages that end early -- the pages of independently cached
 * documents composed into one context ([KV Packet] sections 1 and 3: cached documents reused at
 * new positions without recomputation; the positions come from the rotary page rows). Slot s of
 * logical page n (physical page p) of sequence b is valid iff n * P + s < seq_lens[b] and
 * s < page_fill[p]; seq_lens[b] counts slots, holes included. Summaries, the tail refresh and
 * attention skip the other slots; kvsel_check_inputs reports an entry outside [1, P]
 * (KVSEL_CHECK_PAGE_FILL). kvsel_append_kv ignores page_fill: the page it writes, a sequence's
 * last, must be full-capacity (page_fill P). NULL: every page holds P valid slots. */

/* max_seq_len: page tables are usually allocated for the longest context a sequence may reach,
 * while the lengths live on the device. A non-zero max_seq_len tells the library how many pages
 * are live at most, ceil(max_seq_len / page_size) (capped at max_pages_per_seq), so launch grids
 * and per-thread key counts follow the live length, not the table width; strides (page table,
 * summaries, score rows) stay max_pages_per_seq. Logical pages at or past that bound are never
 * summarized, scored or selected: a longer sequence is selected over as if it held its first
 * max_seq_len tokens, and kvsel_check_inputs reports it (KVSEL_CHECK_SEQ_LEN). Attention over a
 * caller-given list reads every listed page the table holds. kvsel_append_kv ignores the bound
 * (it needs room in the table only). 0 means max_pages_per_seq * page_size. */

/* Host struct: rotary re-positioning of keys ([KV Packet] section 1). Rotate-half convention:
 * channel pair (i, i + D/2) with c = cos[row][i], s = sin[row][i] becomes
 * (x_i*c - x_{i+D/2}*s, x_{i+D/2}*c + x_i*s), each product and sum rounded to fp32 separately
 * (no fused multiply-add), then rounded to the element type (round-to-nearest-even).
 * Slot s of physical page p uses table row page_row[p] + row_step * s; page_row[p] < 0 leaves
 * the page as it is. row_step 1 encodes per-token positions; row_step 0 shifts a whole page.
 * per_sequence != 0: page_row is [B][max_pages_per_seq] and logical page n of sequence b uses
 * page_row[b][n] instead, so sequences that share a document's pages can place it at different
 * positions (composed contexts); kvsel_rope_shift, which rewrites physical pages, rejects it
 * (KVSEL_ERR_UNSUPPORTED). */
typedef struct kvsel_rope {
  const float* cos;        /* [n_rows][D/2] fp32                                       */
  const float* sin;        /* [n_rows][D/2] fp32                                       */
  const int32_t* page_row; /* [num_phys_pages], or [B][max_pages_per_seq] (per_sequence);
                              every used row must be < n_rows                           */
  int32_t n_rows;
  int32_t row_step;        /* 0 or 1                                                    */
  int32_t per_sequence;    /* 0: rows by physical page; 1: by (sequence, logical page)  */
} kvsel_rope;

/* Host struct: speculative reuse with correction ([FreeKV] section 2.1). For every (b, j):
 * C = mean over the G query heads of KV head j of cos(q[b][h], q_prev[b][h]), computed in fp64;
 * corrected = first_step || C < tau (strict); the list used for attention is the fresh
 * selection of this call when corrected, else prev_idx / prev_cnt (the previous step's fresh
 * selection). */
typedef struct kvsel_reuse {
  const void* q_prev;       /* [B][Hq][D] element type: previous step's query           */
  const int32_t* prev_idx;  /* [B][Hkv][k]                                              */
  const int32_t* prev_cnt;  /* [B][Hkv]                                                 */
  double tau;
  int32_t first_step;       /* non-zero: always use the fresh selection                */
  int32_t* used_idx;        /* out [B][Hkv][k]                                          */
  int32_t* used_cnt;        /* out [B][Hkv]                                             */
  uint8_t* corrected;       /* out [B][Hkv], 1 = fresh selection used                   */
  double* similarity;       /* out [B][Hkv], may be NULL                                */
} kvsel_reuse;

/* ABI version (KVSEL_ABI_VERSION of the build). */
int32_t kvsel_abi_version(void);

/* Static string naming a status code; never NULL. */
const char* kvsel_status_str(kvsel_status status);

/* Bytes of device workspace `op` needs for this cache descriptor, top-k size k and (for
 * KVSEL_OP_ATTENTION) pages_per_split (0 = the library's choice). Returns 0 for invalid input.
 * Pure host arithmetic: touches no device.
 * A workspace may be reused by later calls on the same stream; two calls in flight at once must
 * not share one. */
size_t kvsel_workspace_bytes(const kvsel_paged_kv* kv, int32_t k, int32_t op,
                             int32_t pages_per_split);

/* Pages per split of the attention that kvsel_select_attend, kvsel_select_attend_static and
 * kvsel_speculative_step run: 4 (the split their fused launches are built for) below 64
 * (sequence, KV head) lists, the default split of kvsel_sparse_decode_attn from 64 lists on; as
 * kvsel_sparse_decode_attn resolves a request, so possibly larger when k needs it. Those calls
 * equal kvsel_sparse_decode_attn at this pages_per_split bit for bit. Returns 0 for invalid input.
 * Pure host arithmetic: touches no device. */
int32_t kvsel_step_pages_per_split(const kvsel_paged_kv* kv, int32_t k);

/* Page-summary build. For every logical page n < N_b of every sequence b and every KV head j,
 * writes summ[b][j][n][0][:] = channel-wise minimum and summ[b][j][n][1][:] = channel-wise
 * maximum of the valid slots' keys of physical page page_table[b][n]. summ is
 * [B][Hkv][max_pages_per_seq][2][D] in the element type (sequence-major: scoring reads a list's
 * summaries as one contiguous run, without the page table); entries n >= N_b are left untouched.
 * tail_only != 0 rebuilds only each sequence's last logical page (the page a decode step appends
 * to). rope != NULL applies the rotary rotation to each key before the reduction (bit-identical
 * to rotating the pool first with kvsel_rope_shift).
 * fp8 cache: the extremes of the dequantized keys (code value * the tile's k_scale, exact),
 * rounded outward to bfloat16 (lo toward -inf, hi toward +inf), so the page score below still
 * bounds q.k over the page's keys; kvsel_score_topk's tail refresh does the same.
 * [FreeKV] section 2.1 chooses KV pages with the query; the min/max page summary is this
 * library's rule for it (the pages do not define one). */
kvsel_status kvsel_build_summaries(const kvsel_paged_kv* kv, const kvsel_rope* rope,
                                   int32_t tail_only, void* summ, void* stream);

/* Query-aware page scoring and top-k selection, per (sequence, KV head).
 * score[b][j][n] = fp32 rounding of the fp64 sum over the G query heads g of KV head j and the D
 * channels d of (q[b][jG+g][d] >= 0 ? q*hi : q*lo) with lo/hi = summ[b][j][n]
 * (an upper bound of sum_g q_g . k over the page's keys). Products are exact in fp64 and the sum
 * is accumulated in fp64.
 * sel_idx[b][j][0..cnt) (int32 [B][Hkv][k]) receives the min(k, N_b) logical pages with the
 * largest scores, ties to the lower page index, listed in ascending page order; the rest of the
 * row is -1. sel_cnt[b][j] (int32 [B][Hkv]) receives the count.
 * scores (fp32 [B][Hkv][max_pages_per_seq], may be NULL) receives the scores of n < N_b.
 * reuse (may be NULL) adds the speculative-reuse decision described at kvsel_reuse, evaluated on
 * this call's fresh selection.
 * flags: KVSEL_SCORE_REFRESH_TAIL first rebuilds summ for each sequence's last logical page from
 * the key pool (rotated by `rope` when non-NULL), exactly as kvsel_build_summaries with
 * tail_only would, and scores that page from the fresh values (the decode-append step).
 * Without the flag summ is only read and rope is ignored.
 * ws / ws_bytes: with scores == NULL, a device workspace of at least
 * kvsel_workspace_bytes(kv, k, KVSEL_OP_SCORE_TOPK, 0) bytes holds the scores; otherwise unused.
 * [FreeKV] sections 1 and 2.1. */
kvsel_status kvsel_score_topk(const kvsel_paged_kv* kv, const kvsel_rope* rope, void* summ,
                              const void* q, int32_t k, int32_t flags, int32_t* sel_idx,
                              int32_t* sel_cnt, float* scores, const kvsel_reuse* reuse, void* ws,
                              size_t ws_bytes, void* stream);

/* Sparse paged decode attention over the selected pages.
 * For every sequence b and query head h (KV head j = h / G), over the valid slots t of the
 * logical pages sel_idx[b][j][0..sel_cnt[b][j]):
 *   z_t = scale * q[b][h] . k_t,  out[b][h] = sum_t softmax(z)_t v_t,  lse[b][h] = log sum exp z
 * with fp32 arithmetic (K/V read in the element type). out is [B][Hq][D] in the element type;
 * lse is fp32 [B][Hq] and may be NULL. A (b, h) with nothing selected gets out = 0 and
 * lse = -inf. The work is split over groups of pages_per_split consecutive selected pages
 * (0 = the library's choice: 8 from 64 lists on; below that 2 when lists x ceil(k / 2) <= 256,
 * about one block per compute unit, else 4; a request is rounded to a supported size, and raised
 * so that a list has at most 256 splits) and the splits are merged by log-sum-exp in a second
 * launch. The default depends on the list count, and the split fixes the order in which the
 * partial sums are combined, so a sequence's outputs may differ in the last bits between batches;
 * a caller that needs batch-independent bits passes pages_per_split.
 * rope != NULL rotates each key on the fly (bit-identical to a pool rotated by kvsel_rope_shift).
 * fp8 cache: k_t and v_t are the dequantized values (code * the page's k_scale / v_scale); the
 * logits take the key scale as scale * k_scale in fp32, and each probability enters the value
 * product as bfloat16(p * v_scale) while the softmax sum adds bfloat16(p).
 * ws / ws_bytes: workspace of kvsel_workspace_bytes(kv, k, KVSEL_OP_ATTENTION, pages_per_split)
 * bytes for the split partials (0 bytes, and ws may be NULL, when there is a single split).
 * [FreeKV] section 2.1 (attention over the retrieved pages), [KV wiki] (decode attention, GQA). */
kvsel_status kvsel_sparse_decode_attn(const kvsel_paged_kv* kv, const kvsel_rope* rope,
                                      const void* q, const int32_t* sel_idx,
                                      const int32_t* sel_cnt, int32_t k, float scale,
                                      int32_t pages_per_split, void* out, float* lse, void* ws,
                                      size_t ws_bytes, void* stream);

/* Selection and attention in one call: the outputs of kvsel_score_topk (without reuse, scores
 * kept in the workspace) followed by kvsel_sparse_decode_attn with pages_per_split =
 * kvsel_step_pages_per_split(kv, k), bit for bit. The top-k is re-derived inside the attention launch by every block of a list from
 * the page scores (each block keeps the pages of its own split), so the K / V reads follow one
 * memory round trip after the scores instead of the selection-ids -> page-table chain, and no
 * separate top-k launch runs. The fused form is taken where it measured faster than the
 * separate launches: fewer than 64 (sequence, KV head) lists, tables of at most 1024 entries
 * (512 for bf16 with P 16) and k up to 1024; other cases run the two calls' launches inside this
 * call. The outputs are the same either way.
 * sel_idx / sel_cnt: as kvsel_score_topk. out / lse: as kvsel_sparse_decode_attn. flags: as
 * kvsel_score_topk. ws / ws_bytes: kvsel_workspace_bytes(kv, k, KVSEL_OP_SELECT_ATTEND, 0).
 * [FreeKV] sections 1 and 2.1. */
kvsel_status kvsel_select_attend(const kvsel_paged_kv* kv, const kvsel_rope* rope, void* summ,
                                 const void* q, int32_t k, int32_t flags, float scale,
                                 int32_t* sel_idx, int32_t* sel_cnt, void* out, float* lse,
                                 void* ws, size_t ws_bytes, void* stream);

/* kvsel_select_attend without a workspace argument, for callers that cannot allocate device
 * memory (code being captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation): the scores and split partials live in a device array of the library
 * (KVSEL_STATIC_SCRATCH_BYTES, one per GPU, held until the process ends). Same outputs as
 * kvsel_select_attend, bit for bit; the call allocates and frees nothing. A call that needs more
 * than KVSEL_STATIC_SCRATCH_BYTES (kvsel_workspace_bytes(kv, k, KVSEL_OP_SELECT_ATTEND, 0))
 * returns KVSEL_ERR_SCRATCH before anything is enqueued. Nothing in the array needs to start at
 * zero (every byte read is written earlier in the same call). Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (several streams, or several threads) race and must
 * be serialized by the caller. The first call on a device looks up the array's device address
 * (hipGetSymbolAddress, with that device current), so it should not be the first call made
 * inside a stream capture. */
kvsel_status kvsel_select_attend_static(const kvsel_paged_kv* kv, const kvsel_rope* rope,
                                        void* summ, const void* q, int32_t k, int32_t flags,
                                        float scale, int32_t* sel_idx, int32_t* sel_cnt, void* out,
                                        float* lse, void* stream);

/* Rotary table: cos[r][i], sin[r][i] (fp32 [n_rows][D/2]) of the angle
 * (first_position + r) * theta^(-2i/D), evaluated in fp64 and rounded to fp32. head_dim is even
 * and <= 128. The D/2 frequencies theta^(-2i/D) are evaluated once on the host with the C
 * library's pow; angles and their cos / sin are evaluated on the device.
 * [KV Packet] section 1 (RoPE encodes position by rotation). */
kvsel_status kvsel_rope_table(double theta, int32_t head_dim, int32_t first_position,
                              int32_t n_rows, float* cos, float* sin, void* stream);

/* Materialized rotary re-positioning: writes the rotated keys of every physical page with
 * page_row[p] >= 0 into k_out ([num_phys_pages][Hkv][P][D], element type) and copies the other
 * pages unchanged. k_out may equal kv->k_pool (in place; unrotated pages are then skipped).
 * Only the pool fields of kv (dtype, num_kv_heads, head_dim, page_size, num_phys_pages,
 * k_pool) are read, but kv must still pass the descriptor checks.
 * [KV Packet] section 1. */
kvsel_status kvsel_rope_shift(const kvsel_paged_kv* kv, const kvsel_rope* rope, void* k_out,
                              void* stream);

/* Speculative decode step: the outputs of kvsel_score_topk with `reuse` (required) followed by
 * kvsel_sparse_decode_attn over the used pages (reuse->used_idx / used_cnt) with pages_per_split
 * = kvsel_step_pages_per_split(kv, k), bit for bit. The attention over the previous step's pages (reuse->prev_idx /
 * prev_cnt), which does not depend on this step's selection, runs in the same launch as the page
 * scoring and the reuse decision; the next launch selects, and re-attends only the lists the
 * decision corrected, over their fresh pages; a last launch merges the splits. With
 * reuse->first_step every list is corrected and no attention runs over the previous pages.
 * Page tables wider than 8192 entries (4096 for bf16 with P 16), k above 1024 and composed
 * sequences (page_fill set) run the two calls serially instead, with the same outputs. One stream; capturable in a HIP graph.
 * sel_idx / sel_cnt and reuse->used_idx / used_cnt must not alias reuse->prev_idx / prev_cnt.
 * ws / ws_bytes: kvsel_workspace_bytes(kv, k, KVSEL_OP_SPECULATIVE_STEP, 0). Other arguments as
 * kvsel_score_topk and kvsel_sparse_decode_attn.
 * [FreeKV] section 2.1 (speculative retrieval: attention at step i over the pages chosen at step
 * i-1, overlapped with the selection; fine-grained correction when the group-mean similarity is
 * below tau). */
kvsel_status kvsel_speculative_step(const kvsel_paged_kv* kv, const kvsel_rope* rope, void* summ,
                                    const void* q, int32_t k, int32_t flags, float scale,
                                    const kvsel_reuse* reuse, int32_t* sel_idx, int32_t* sel_cnt,
                                    void* out, float* lse, void* ws, size_t ws_bytes,
                                    void* stream);

/* Quantize a cache's pages to fp8 (the pages name a quantized cache only as a trade-off of
 * capacity against a little accuracy -- [KV wiki], Contradictions & Updates entry -- and fix no
 * format; this library's rule): for every physical page p and KV head j, of K and of V
 * separately, scale[p][j] = amax / 448 in fp32 (amax = the largest magnitude of the tile's P * D
 * values; 1 when it is 0), and every value x becomes the OCP FP8 E4M3 code of fp32(x / scale)
 * (fp32 division, correctly rounded), rounded to nearest with ties to an even mantissa and
 * magnitudes from 448 up saturating to 448; the sign bit is kept.
 * src: a KVSEL_F32 or KVSEL_BF16 cache; its page table and lengths are not used. k_codes:
 * [num_phys_pages][Hkv][P][D] uint8 and k_scale [num_phys_pages][Hkv] fp32 out; v_codes
 * ([num_phys_pages][Hkv][D][P], the device value layout) and v_scale likewise from src->v_pool,
 * both NULL to quantize K only. The outputs make an fp8 descriptor with the same page table.
 * One launch; one wave per tile. */
kvsel_status kvsel_quantize_pages(const kvsel_paged_kv* src, uint8_t* k_codes, float* k_scale,
                                  uint8_t* v_codes, float* v_scale, void* stream);

/* Device-side free-page list for kvsel_append_kv (the caller's page pool, kept on the device so
 * that a captured decode loop needs no host step to grow a sequence): ids[0 .. *count) are free
 * physical page ids; a token that opens a page takes the top one, ids[*count - 1], and
 * decrements *count. The library never pushes ids back: refill the list and set *count between
 * calls. */
typedef struct kvsel_free_pages {
  int32_t* ids;      /* device int32 [capacity] */
  int32_t* count;    /* device int32 [1], 0 <= *count <= capacity */
  int32_t capacity;  /* host: entries of ids (>= 1) */
} kvsel_free_pages;

/* Decode-time append ([KV wiki]: a decode step stores the new token's key and value and keeps
 * every earlier one). For every sequence b with L = seq_lens[b] in [0, max_pages_per_seq * P):
 * writes k_new[b][j][:] into slot L % P of logical page L / P (physical page
 * page_table[b][L / P]) of the key pool and v_new[b][j][:] into the same slot of the value pool,
 * for every KV head j; when summ is non-NULL, keeps that page's summary current: a token that
 * opens a page (L % P == 0) sets lo = hi = its key, any other takes lo = min(lo, key),
 * hi = max(hi, key) -- equal to kvsel_build_summaries' rebuild of the page when the summary was
 * current before the call; then writes seq_lens_out[b] = L + 1.
 * A sequence with no room (L == max_pages_per_seq * P) or L < 0 is left unchanged and, when flags
 * is non-NULL, KVSEL_CHECK_SEQ_LEN is ORed into *flags (device uint32).
 * The page a token opens: with free_pages NULL, the table entry is the caller's allocator's to set
 * before the call (an entry outside the pool is clamped into it, as by every reader). With a
 * free-page list, the token takes a page from it and page_table[b][L / P] is set to that page;
 * which sequence gets which of the taken ids is unspecified when several open a page in one call.
 * If the list is empty the sequence is left unchanged and KVSEL_CHECK_NO_FREE_PAGE is ORed into
 * *flags; an id outside [0, num_phys_pages) (or *count > capacity) is consumed, the sequence left
 * unchanged and KVSEL_CHECK_PAGE_ID ORed in.
 * kv->k_pool, kv->v_pool (and, with a free list, kv->page_table) are written despite the
 * descriptor's const qualifiers. Keys are stored as given: with a rotary gather, store keys
 * already at their positions, on pages whose page_row is -1.
 * k_new, v_new: [B][Hkv][D] element type. seq_lens_out: int32 [B], may equal kv->seq_lens (in
 * place). summ: [B][Hkv][max_pages_per_seq][2][D] as kvsel_build_summaries writes it, or NULL.
 * One launch of one block per sequence. */
kvsel_status kvsel_append_kv(const kvsel_paged_kv* kv, const void* k_new, const void* v_new,
                             void* summ, int32_t* seq_lens_out,
                             const kvsel_free_pages* free_pages, uint32_t* flags, void* stream);

/* Device-side check of the contents every other entry point takes on trust (the host cannot
 * read device memory before enqueuing): ORs into *flags (device uint32, sticky: bits are set,
 * never cleared by the library)
 *   KVSEL_CHECK_SEQ_LEN   if some seq_lens[b] < 0 or > the live bound (max_seq_len if non-zero,
 *                         else max_pages_per_seq * page_size);
 *   KVSEL_CHECK_PAGE_ID   if some page_table[b][n], n < N_b, is outside [0, num_phys_pages);
 *   KVSEL_CHECK_PAGE_FILL with page_fill, if such a page's page_fill is outside [1, P];
 *   KVSEL_CHECK_SELECTION (only when sel_idx != NULL; sel_cnt and k then required) if some
 *     sel_cnt[b][j] is outside [0, min(k, N_b)] or the first sel_cnt[b][j] entries of
 *     sel_idx[b][j] are not strictly ascending page ids in [0, N_b).
 * Reads stay inside the arrays the descriptor sizes whatever their contents, so it is safe to
 * run on the inputs it is meant to reject. One launch of one block per sequence; for debugging
 * and input validation, not for the decode path. */
#define KVSEL_CHECK_SEQ_LEN 1u
#define KVSEL_CHECK_PAGE_ID 2u
#define KVSEL_CHECK_SELECTION 4u
#define KVSEL_CHECK_NO_FREE_PAGE 8u /* kvsel_append_kv only: the free-page list was empty */
#define KVSEL_CHECK_PAGE_FILL 16u   /* some page_fill[p], p referenced, outside [1, P] */
kvsel_status kvsel_check_inputs(const kvsel_paged_kv* kv, const int32_t* sel_idx,
                                const int32_t* sel_cnt, int32_t k, uint32_t* flags, void* stream);

/* ---- measurement ---- */

/* Read-bandwidth probe: gathers n_chunks chunks of chunk_bytes bytes (1, 2, 4, 8, 16 or 32 KiB;
 * each chunk 16-byte aligned) whose device addresses are in chunk_addr (device array, uint64
 * [n_chunks]), one wave per chunk with every load issued before the first use, and folds the
 * data into *sink (device, one word; written only in the practically impossible case that the
 * fold equals a fixed constant). Given the K and V tiles an attention call reads, it times the
 * same bytes moved with no index chain, arithmetic or merge: context for the attention
 * kernel's bandwidth, not part of the decode path.
 * [KV wiki] (decode speed is set by memory bandwidth). */
kvsel_status kvsel_gather_probe(const uint64_t* chunk_addr, int32_t n_chunks, int32_t chunk_bytes,
                                uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVSEL_H */
