/*
 * ra.h -- C ABI of the per-rank blockwise Ring Attention library (gfx950 / MI355X).
 *
 * One rank of Ring Attention keeps its query chunk fixed and folds in the c key/value
 * blocks of the ring, one per round, with the online softmax: a running maximum and a
 * running sum per query row, and a partial output rescaled whenever the maximum grows.
 * The result equals softmax attention over the full row ("Ring Attention and Ulysses
 * shard a sequence two different ways, ...", section "Ring Attention: point-to-point
 * rotation, and an online softmax that never sees the whole row at once"; "What do you
 * do about long sequences and sparse models?", section "How does attention survive
 * being split?"). On one GPU the c rounds are replayed in ring order from KV blocks
 * that already sit in device memory.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers. The caller allocates and frees every
 *     buffer; the library allocates nothing and keeps no device state.
 *   - Tensors are dense and row-major with the head dimension innermost. Base pointers
 *     of q, k_blocks, v_blocks and out tensors must be 16-byte aligned; lse arrays
 *     4-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work is
 *     enqueued on it and the call returns without waiting.
 *   - Every argument is checked on the host before anything is enqueued. A nonzero
 *     return means nothing was enqueued and no output was touched; ra_last_error()
 *     then describes the problem. Inputs are not checked for NaN or infinity; results
 *     for non-finite inputs are unspecified.
 *   - Calls are reentrant; the last-error text is per host thread. Nothing is
 *     synchronized or allocated, so calls on different streams may run at once and a
 *     sequence of calls may be captured in a HIP graph and replayed.
 *   - Output buffers must not overlap any input buffer (RA_ERR_ARG), except where an
 *     entry point says otherwise (ra_merge's in-place update).
 */
#ifndef RA_H
#define RA_H

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k_blocks, v_blocks and out. Accumulation is always fp32. */
enum ra_dtype { RA_BF16 = 0, RA_F32 = 1 };

/* Return codes. */
enum ra_status {
  RA_OK = 0,
  RA_ERR_ARG = -1,         /* null pointer, c < 1, rank outside [0, c), hq % hkv != 0,
                              negative size, bad round range, unknown dtype, outputs
                              overlapping inputs */
  RA_ERR_SHAPE = -2,       /* causal with nq != nkv; causal zigzag with odd nkv;
                              c * nkv above 2^30 tokens, a KV head slab (nkv rows of
                              head_dim elements) above 2^31-1 bytes, or more than
                              2^31-1 tiles */
  RA_ERR_UNSUPPORTED = -3, /* (dtype, head_dim) pair not built: bf16 takes d = 64 or
                              128; fp32 takes d = 8, 16, ..., 128 */
  RA_ERR_ALIGN = -4,       /* a base pointer not 16-byte aligned */
  RA_ERR_LAUNCH = -5       /* the HIP runtime refused the launch */
};

/*
 * ra_rank_forward -- one rank's share of Ring Attention, folding in the KV blocks of
 * rounds [round_begin, round_end) in ring order.
 *
 * Round r uses KV block (rank - r) mod c: round 0 is the rank's own block and every
 * later round the block that has travelled one more hop, since rank i sends to rank
 * i+1 (the sections cited above). round_begin = 0, round_end = c folds the whole ring
 * in one launch ("fused"); a shorter range gives the partial result of those rounds,
 * which ra_merge combines with others.
 *
 *   q         [batch, hq, nq, head_dim]          the rank's queries
 *   k_blocks  [c, batch, hkv, nkv, head_dim]     KV block j = rank j's keys, owner order
 *   v_blocks  [c, batch, hkv, nkv, head_dim]     (same layout)
 *   out       [batch, hq, nq, head_dim]          written, element type = dtype:
 *             softmax(q k^T / sqrt(head_dim) + mask) v over the keys of the folded
 *             blocks, already divided by the row sum; 0 for a row with no allowed key
 *   lse       [batch, hq, nq] fp32, or NULL to skip: natural log of the sum of
 *             exp(q.k / sqrt(head_dim)) over the allowed keys; -inf for a row with
 *             no allowed key
 *
 *   hkv       KV heads; query head h reads KV head h / (hq / hkv) (grouped-query
 *             attention, "What do you do about long sequences and sparse models?",
 *             section "Why did Llama 3 not use a ring?")
 *   causal    nonzero: key position j is visible to query position i iff j <= i
 *             ("Context & Expert Parallelism", section "Context parallelism: splitting
 *             the sequence"). Needs nq == nkv.
 *   zigzag    with causal: the sequence is cut into 2c chunks of nkv/2 tokens and
 *             owner i (the rank for q, block j's owner for k/v) holds chunk i in rows
 *             [0, nkv/2) and chunk 2c-1-i in rows [nkv/2, nkv) ("What do you do about
 *             long sequences and sparse models?", section "What breaks the load
 *             balance?"). Without zigzag owner i holds chunk i of c. Ignored when
 *             causal is zero (positions then play no part).
 *   Tiles of keys that no query of a tile may see are never loaded or computed.
 *
 * nq = 0 or batch = 0 enqueues nothing and returns RA_OK. nkv = 0 (non-causal) or an
 * empty round range writes out = 0 and lse = -inf. Pointers of empty tensors may be
 * NULL. out and lse must not overlap each other or any input (RA_ERR_ARG).
 */
int ra_rank_forward(const void* q, const void* k_blocks, const void* v_blocks,
                    void* out, float* lse,
                    int batch, int hq, int hkv, int nq, int nkv, int head_dim,
                    int c, int rank, int causal, int zigzag,
                    int round_begin, int round_end,
                    int dtype, void* stream);

/*
 * ra_rank_forward_doc -- ra_rank_forward (always causal) with the document mask of a
 * packed sequence: attention does not cross document boundaries, the mask Llama 3's
 * all-gather context parallelism was chosen to support ("What do you do about long
 * sequences and sparse models?", section "Why did Llama 3 not use a ring?").
 *
 *   doc_start [c * nkv] int32, device: for every global token position p, the position
 *             where p's document begins (documents are contiguous spans, so the value
 *             also identifies the document). The query at position p sees exactly
 *             the keys at positions x with doc_start[p] <= x <= p. Any int32 values
 *             are accepted with that meaning (a value above p leaves the row without
 *             keys: out = 0, lse = -inf). Positions are those of ra_rank_forward
 *             (zigzag or contiguous ownership of the sequence of c * nkv tokens).
 *             Read-only; 4-byte aligned; must not be NULL unless batch or nq is 0.
 *
 * Every other argument, the layouts, outputs and errors are those of ra_rank_forward
 * with causal = 1. Tiles of keys that lie before every document start of a query
 * tile, or after its last query, are never loaded or computed.
 */
int ra_rank_forward_doc(const void* q, const void* k_blocks, const void* v_blocks,
                        const int* doc_start, void* out, float* lse,
                        int batch, int hq, int hkv, int nq, int nkv, int head_dim,
                        int c, int rank, int zigzag,
                        int round_begin, int round_end,
                        int dtype, void* stream);

/*
 * ra_rank_forward_accumulate -- ra_rank_forward (or, with doc_start, ra_rank_forward_doc)
 * over rounds [round_begin, round_end) whose result is folded into the running result
 * already held in (out, lse) instead of overwriting it. This is one step of the streamed
 * ring: each round's partial joins the accumulator as its block arrives, combined
 * exactly through the maxima and sums of both ("What do you do about long sequences and
 * sparse models?", section "How does attention survive being split?"), with no separate
 * merge launch or partial buffer.
 *
 *   out [batch, hq, nq, head_dim], element type out_dtype, device: in, the running
 *       output; out, the output over the union of its keys and this call's. Where the
 *       incoming lse is -inf the incoming out is ignored (it may hold anything, NaN
 *       included).
 *   out_dtype: the running output's element type: dtype, or RA_F32 with bf16 inputs.
 *       Every call rounds the running output to its type, so a bf16 one gains up to
 *       half a bf16 ulp per call (a few ulps over a long ring); an fp32 one keeps the
 *       streamed result as close to the fused one as fp32 allows.
 *   lse [batch, hq, nq] fp32, device: in, the running lse (set it to -inf before the
 *       first call); out, the lse over the union. Must not be NULL.
 *   doc_start: NULL for no document mask, else as in ra_rank_forward_doc (then causal
 *       must be 1).
 *
 * The folded result equals ra_merge of the accumulator with this call's ra_rank_forward
 * result: for M = max(lse_old, lse_new), M = -inf gives out = 0 and lse = -inf; else
 * w = e^(lse - M) for each side, out = (w_old out_old + w_new out_new) / (w_old + w_new),
 * lse = M + ln(w_old + w_new). The call's rounds must hold keys disjoint from those
 * already folded in (a ring visits each block once). Every other argument, layout and
 * error is that of ra_rank_forward, plus RA_ERR_ARG for a NULL lse, for doc_start with
 * causal = 0, or for an out_dtype other than dtype or (bf16 inputs) RA_F32. Rows to
 * which the call's rounds contribute no key keep their (out, lse) when the running lse
 * is finite. An empty round range leaves (out, lse) unchanged.
 */
int ra_rank_forward_accumulate(const void* q, const void* k_blocks, const void* v_blocks,
                               const int* doc_start, void* out, float* lse,
                               int batch, int hq, int hkv, int nq, int nkv, int head_dim,
                               int c, int rank, int causal, int zigzag,
                               int round_begin, int round_end,
                               int dtype, int out_dtype, void* stream);

/*
 * ra_merge -- combine two partial results over disjoint key sets into the result over
 * their union ("What do you do about long sequences and sparse models?", section "How
 * does attention survive being split?": partials combine exactly through their
 * running maximum and sum).
 *
 * For each of `rows` rows with M = max(lse_a, lse_b):
 *   M = -inf            -> out = 0, lse = -inf
 *   otherwise           -> wa = e^(lse_a - M), wb = e^(lse_b - M),
 *                          out = (wa * out_a + wb * out_b) / (wa + wb),
 *                          lse = M + ln(wa + wb)
 *
 *   out_a, out_b, out   [rows, head_dim], element type = dtype (fp32 arithmetic)
 *   lse_a, lse_b, lse   [rows] fp32
 * out may alias out_a or out_b and lse may alias lse_a or lse_b (in-place update).
 * Each merge rounds out to dtype: a long stream of in-place bf16 merges gains up to half
 * a bf16 ulp per merge, which ra_rank_forward_accumulate with an fp32 running output
 * avoids.
 * rows = 0 enqueues nothing and returns RA_OK.
 * Errors: RA_ERR_ARG (null pointer, rows < 0, unknown dtype), RA_ERR_UNSUPPORTED
 * (head_dim not a multiple of 8 in [8, 512]), RA_ERR_ALIGN, RA_ERR_LAUNCH.
 */
int ra_merge(const void* out_a, const float* lse_a, const void* out_b, const float* lse_b,
             void* out, float* lse, long long rows, int head_dim, int dtype, void* stream);

/* Text describing the last nonzero return on the calling host thread ("" if none). */
const char* ra_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int ra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
