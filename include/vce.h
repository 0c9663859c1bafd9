/*
 * vce.h -- vocabulary-sharded LM-head cross-entropy and masked embedding
 *          lookup over one tied table, for AMD Instinct MI355X (gfx950).
 *
 * Sources (page titles):
 *   [VS]  "Vocabulary shards: look up locally and normalize globally"
 *   [SP]  "Sequence-parallel normalization: shard tokens, retain their hidden features"
 *   [PAD] "Training collapses when token embeddings are not padded to a multiple of 64"
 *   [SS]  "Sampled Softmax with Over-Tokenized Transformer"
 *   [TP]  "Tensor Parallelism (TP)" (vLLM on Neuron design notes)
 *
 * Problem statement. Hidden rows h[T,H]; one table W[V_pad,H] shared by the
 * input embedding and the output projection; V_real <= V_pad real classes
 * (rows V_real..V_pad-1 are padding and never classes); num_shards contiguous
 * equal row ranges of S = V_pad / num_shards rows each ([TP] "Embedding"),
 * shard k owning rows [k*S, (k+1)*S). On one GPU the shards are emulated:
 * every shard computes only with its own rows and the results are merged on
 * the device exactly as a cross-shard reduction would merge them.
 *
 * Conventions for every entry point:
 *   - Every array argument is a DEVICE pointer owned by the caller, row-major
 *     and contiguous. The library allocates no memory, never synchronises the
 *     host, keeps no state between calls and may be called concurrently on
 *     different streams with disjoint outputs and workspaces.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All work is enqueued on it; outputs are valid once it has drained.
 *   - Argument errors are detected on the host and returned BEFORE any HIP
 *     call is made, so they can be tested without a GPU.
 *   - Data-dependent faults are counted, never aborted on: an out-of-range
 *     target or ID is counted in a device scalar and handled by rule.
 *   - Element types: VCE_F32 = IEEE float32, VCE_BF16 = bfloat16 (raw 16-bit
 *     patterns). IDs and targets are int32. Statistics, losses and gradients
 *     are float32.
 *   - Alignment: every array pointer must be 16-byte aligned and H must be a
 *     multiple of 8 (rows are read in 16-byte pieces).
 *   - T = 0 is valid: scalars are written (0), nothing else is touched.
 */
#ifndef VCE_H
#define VCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VCE_OK = 0,
  VCE_ERR_NULL = 1,      /* a required pointer is NULL                          */
  VCE_ERR_SHAPE = 2,     /* T < 0, H <= 0, V_real not in [1, V_pad], ignore_index
                            inside [0, V_real), P < 1, capacity too small, or a
                            size too large for 32-bit indexing of one dimension  */
  VCE_ERR_SHARD = 3,     /* num_shards not in [1, 128], V_pad not a multiple of
                            num_shards, or a malformed shard_rows list          */
  VCE_ERR_DTYPE = 4,     /* unknown element type, reduction or accumulate flag   */
  VCE_ERR_ALIGN = 5,     /* a pointer not 16-byte aligned, or H % 8 != 0         */
  VCE_ERR_WORKSPACE = 6, /* workspace NULL or smaller than the query returned    */
  VCE_ERR_HIP = 7        /* a HIP launch failed (hipGetLastError != success)     */
} vce_status;

typedef enum { VCE_F32 = 0, VCE_BF16 = 1 } vce_dtype;

typedef enum { VCE_REDUCE_MEAN = 0, VCE_REDUCE_SUM = 1 } vce_reduction;

/* Flags of vce_bwd's `accumulate` argument. */
enum { VCE_ACC_DW = 1, VCE_ACC_DH = 2 };

/* Version of this interface (changes when a signature changes). */
int32_t vce_abi_version(void);

/* Human-readable text of a status code (static string, never NULL). */
const char* vce_strerror(vce_status s);

/* ------------------------------------------------------------------------ *
 * Cross-entropy forward.                                                    *
 *                                                                           *
 * [VS] paragraph 3: for every token the logits z[t,v] = h[t,:] . W[v,:] of  *
 * the real rows v < V_real are normalised by one global log-sum-exp built   *
 * from per-shard maxima and sums of exponentials; the target logit comes    *
 * from the single shard that owns the target. [VS] paragraph 4 and [PAD]    *
 * section 5: padded rows are excluded (as if their logits were -inf);       *
 * a target equal to ignore_index contributes no loss. [VS] paragraph 5: the *
 * full [T, V] logits are never stored.                                      *
 *                                                                           *
 * In:  h [T,H] dt, W [V_pad,H] dt, targets [T] int32.                       *
 * Out: lse [T]          log-sum-exp over the real rows (also for ignored     *
 *                       tokens, [SP] paragraph 5);                           *
 *      loss [T]         lse - z[t, y_t] for valid targets, else 0;           *
 *      loss_sum [1]     sum of loss in a fixed order (deterministic);        *
 *      n_valid [1]      number of targets in [0, V_real);                    *
 *      n_bad_target [1] number of targets outside [0, V_real) that are not   *
 *                       ignore_index (treated as ignored);                   *
 *      shard_stats      optional (NULL = not written): float [2][num_shards] *
 *                       [T]: plane 0 the shard maxima m_k (-inf for a shard  *
 *                       with no real row), plane 1 the sums s_k of           *
 *                       exp(z - m_k) over the shard's real rows.             *
 * Rows of W at or past V_real are never read; any bits there (NaN, Inf) do  *
 * not change any output.                                                    *
 * ws: device workspace of at least vce_fwd_workspace_bytes(...) bytes.      *
 * ------------------------------------------------------------------------ */
size_t vce_fwd_workspace_bytes(int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                               int32_t num_shards, vce_dtype dt);

vce_status vce_fwd(const void* h, const void* W, const int32_t* targets,
                   int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                   int32_t num_shards, int32_t ignore_index, vce_dtype dt,
                   float* lse, float* loss, float* loss_sum, int32_t* n_valid,
                   int32_t* n_bad_target, float* shard_stats,
                   void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Cross-entropy backward.                                                   *
 *                                                                           *
 * [VS] paragraph 4: the gradient of a valid logit is its global probability *
 * minus the target indicator, times the loss scaling. Logits are recomputed *
 * tile by tile (never stored whole) to form                                 *
 *   G[t,v] = scale * (exp(z[t,v] - lse[t]) - [v == y_t])                    *
 * for valid targets and real rows, else exactly 0, and then                 *
 *   dh = G W        ([T,H] float32; see accumulate)                         *
 *   dW = G^T h      (rows < V_real; [V_pad,H] float32)                      *
 * scale = grad_loss[0] / max(n_valid[0], 1) for VCE_REDUCE_MEAN ([SP]       *
 * paragraph 3: one average over the valid tokens) or grad_loss[0] for       *
 * VCE_REDUCE_SUM; both scalars are read on the device (no host sync).       *
 * accumulate: a set of VCE_ACC_* flags. Without VCE_ACC_DW every row of   *
 * dW is written (rows >= V_real get 0); with it G^T h is added into rows   *
 * < V_real and rows >= V_real are left unchanged. Without VCE_ACC_DH dh is *
 * overwritten; with it G W is added into dh (a second head's gradient on   *
 * the same hidden rows, [SS] Setup, OT-H). Other bits: VCE_ERR_DTYPE.      *
 * lse must be the forward's output for the same inputs.                    *
 * The vocabulary is processed in chunks: at least two once V_pad spans two *
 * 256-row tiles, each at most 131072 rows; equal groups of whole shards     *
 * when shards fit, else every shard cut into tile-aligned pieces. G of one  *
 * chunk ([T][chunk], never [T][V]) is staged in the workspace in the input  *
 * element type (bf16 rounded to nearest-even, or float32), then dh receives *
 * G_chunk W_chunk (in chunk order) and the chunk's rows of dW receive       *
 * G_chunk^T h. When the tiles of the dh or dW product would leave CUs idle, *
 * its K range is split in 2..8 parts where that is estimated to save time   *
 * (rounds of tiles over 256 CUs against the partial planes' traffic), or,   *
 * for an unsplit dW, only the rows past its whole rounds of tiles are (a    *
 * second launch): the later parts go to float32 partial planes in the       *
 * workspace and are added in a fixed order afterwards (results stay         *
 * deterministic).                                                           *
 * ------------------------------------------------------------------------ */
size_t vce_bwd_workspace_bytes(int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                               int32_t num_shards, vce_dtype dt);

vce_status vce_bwd(const void* h, const void* W, const int32_t* targets, const float* lse,
                   const float* grad_loss, const int32_t* n_valid, vce_reduction red,
                   int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                   int32_t num_shards, int32_t ignore_index, vce_dtype dt,
                   float* dh, float* dW, int32_t accumulate,
                   void* ws, size_t ws_bytes, void* stream);

/* Number of events vce_bwd_timed records for these arguments:
 * 1 + 3 * (number of vocabulary chunks); 0 for invalid arguments. */
int64_t vce_bwd_event_count(int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                            int32_t num_shards, vce_dtype dt);

/* Same as vce_bwd, for profiling tools: when `events` is not NULL it holds
 * n_events == vce_bwd_event_count(...) hipEvent_t handles (passed as void*)
 * created by the caller; they are recorded on `stream`: events[0] before the
 * first kernel, then for chunk c events[1 + 3c] after its G, [2 + 3c] after
 * its dh contribution and [3 + 3c] after its dW rows. A different n_events
 * returns VCE_ERR_SHAPE. With events == NULL this is vce_bwd. */
vce_status vce_bwd_timed(const void* h, const void* W, const int32_t* targets, const float* lse,
                         const float* grad_loss, const int32_t* n_valid, vce_reduction red,
                         int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                         int32_t num_shards, int32_t ignore_index, vce_dtype dt,
                         float* dh, float* dW, int32_t accumulate,
                         void* ws, size_t ws_bytes, void* stream, void* const* events,
                         int64_t n_events);

/* ------------------------------------------------------------------------ *
 * Greedy argmax over the sharded LM head (greedy decoding).                 *
 *                                                                           *
 * [TP] "LM Head (ColumnParallelLinear)": every rank computes the logits of  *
 * its own vocabulary shard, and an on-device sampler finds the global       *
 * argmax across the shards without gathering the [T, V] logits. Here every  *
 * vocabulary tile reduces its logits tile to (largest logit, lowest row     *
 * holding it) over its real rows; the tiles of a shard merge into the       *
 * shard's report, and the shard reports into the global result, always by   *
 * larger value, then lower index (so ties go to the lowest vocabulary       *
 * index, as for an unsharded argmax that returns the first maximum).        *
 * Padded rows are never read and never chosen ([VS] paragraph 4).           *
 *                                                                           *
 * In:  h [T,H] dt, W [V_pad,H] dt.                                          *
 * Out: index [T] int32   argmax over v < V_real of z[t,v] = h[t,:].W[v,:];  *
 *      value [T] float   that logit (float32 accumulation);                 *
 *      shard_value, shard_index: optional (NULL = not written) [num_shards] *
 *                        [T] float / int32, each shard's report (-inf and   *
 *                        -1 for a shard that owns no real row).             *
 * ws: device workspace of at least vce_argmax_workspace_bytes(...) bytes.   *
 * Errors as for vce_fwd.                                                    *
 * ------------------------------------------------------------------------ */
size_t vce_argmax_workspace_bytes(int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                                  int32_t num_shards, vce_dtype dt);

vce_status vce_argmax(const void* h, const void* W, int64_t T, int64_t H, int64_t V_real,
                      int64_t V_pad, int32_t num_shards, vce_dtype dt, int32_t* index,
                      float* value, float* shard_value, int32_t* shard_index,
                      void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Masked embedding lookup.                                                  *
 *                                                                           *
 * [VS] paragraph 1: a shard tests whether an ID is in its row range, turns  *
 * owned IDs into local indices and contributes the row; non-owners give     *
 * zero and the sum over shards is the embedding. [VS] paragraph 2: the      *
 * table is never indexed with an unmasked global ID. Rule for IDs outside   *
 * [0, V_real) (negative, padded rows, >= V_pad): a zero row, counted in     *
 * n_bad_id. Each output row is a bit-exact copy of its owner's row          *
 * (the owner's row is selected, not added to zeros, so -0.0 is kept).       *
 * In:  ids [T] int32, W [V_pad,H] dt.  Out: out [T,H] dt,                   *
 *      n_bad_id [1] int32 (optional, NULL = not counted).                   *
 * ------------------------------------------------------------------------ */
vce_status vemb_fwd(const int32_t* ids, const void* W, int64_t T, int64_t H,
                    int64_t V_real, int64_t V_pad, int32_t num_shards, vce_dtype dt,
                    void* out, int32_t* n_bad_id, void* stream);

/* ------------------------------------------------------------------------ *
 * Embedding backward (scatter-add).                                         *
 *                                                                           *
 * [VS] paragraph 2: repeated occurrences of one token add their gradients   *
 * into the one row that owns it; with a tied table every contribution lands *
 * in the same tensor. dW[v,:] (+)= sum of dout[t,:] over t with ids[t] == v, *
 * for v < V_real, summed in float32 in a fixed order (deterministic, one   *
 * writer per row): in increasing t, or, for an ID with 64 or more tokens,   *
 * 16 running sums over every 16th token added in order. IDs outside         *
 * [0, V_real) are dropped.                                                  *
 * accumulate = 1: add into the touched rows only (e.g. after vce_bwd wrote  *
 * the LM-head part of a tied dW); accumulate = 0: the whole table is        *
 * overwritten (untouched rows become 0).                                    *
 * In: ids [T] int32, dout [T,H] of dout_dt.  Out: dW [V_pad,H] float32.     *
 * ------------------------------------------------------------------------ */
size_t vemb_bwd_workspace_bytes(int64_t T, int64_t H, int64_t V_real, int64_t V_pad);

vce_status vemb_bwd(const int32_t* ids, const void* dout, vce_dtype dout_dt,
                    int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                    int32_t num_shards, float* dW, int32_t accumulate,
                    void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Hashed n-gram input embedding (the Over-Tokenized input side).           *
 *                                                                           *
 * [SS] Setup and its loss listing: to the embedding of every input token    *
 * OT adds a hashed 2-gram and a hashed 3-gram embedding of the n-grams that *
 * end at that token:                                                        *
 *   out[t] = E[ids[t]] + E2[row2(t)] + E3[row3(t)]                          *
 * row2(t) = mix64(ids[t-1]*V_real + ids[t]) mod rows2 and                   *
 * row3(t) = mix64((ids[t-2]*V_real + ids[t-1])*V_real + ids[t]) mod rows3   *
 * (unsigned 64-bit; mix64 = the SplitMix64 output finaliser, Steele, Lea &  *
 * Flood 2014). The page gives no hash; this is the library's choice. An     *
 * n-gram exists only when t >= n-1 and all its IDs are in [0, V_real); a    *
 * missing n-gram, like an invalid unigram ID, adds a zero row. The T tokens *
 * form one sequence. Each table is split into num_shards contiguous equal   *
 * shards (V_pad, rows2 and rows3 multiples of num_shards) and read by owner *
 * and local index, as vemb_fwd reads E. The three rows are added in float32 *
 * in that order and stored in dt (bf16 rounded to nearest-even).            *
 *                                                                           *
 * In:  ids [T] int32; E [V_pad,H], E2 [rows2,H], E3 [rows3,H] dt.          *
 * Out: out [T,H] dt; ids2, ids3 [T] int32: row2(t) / row3(t), -1 where the  *
 *      n-gram is missing (the backward is vemb_bwd with these as IDs and    *
 *      rows2 / rows3 as V_real = V_pad); n_bad_id [1] (optional) as vemb_fwd.*
 * rows2, rows3 in [1, 2^31); errors as for vemb_fwd.                        *
 * ------------------------------------------------------------------------ */
vce_status vngram_fwd(const int32_t* ids, const void* E, const void* E2, const void* E3,
                      int64_t T, int64_t H, int64_t V_real, int64_t V_pad, int64_t rows2,
                      int64_t rows3, int32_t num_shards, vce_dtype dt, void* out,
                      int32_t* ids2, int32_t* ids3, int32_t* n_bad_id, void* stream);

/* ------------------------------------------------------------------------ *
 * Greedy argmax without a workspace, for callers that cannot allocate        *
 * device memory (code under HIP graph capture, tight serving loops).         *
 *                                                                           *
 * The same call as vce_argmax (same kernels, arguments, results and errors) *
 * except that the per-tile reports live in a static device buffer of the    *
 * library, 16 MiB (VCE_NOALLOC_SCRATCH_BYTES) on each GPU it runs on, held  *
 * until the process ends. Its address is looked up once per device on the  *
 * first call with that device current. Allocates nothing.                   *
 * Errors: as vce_argmax; VCE_ERR_WORKSPACE when vce_argmax_workspace_bytes  *
 * for the same arguments exceeds VCE_NOALLOC_SCRATCH_BYTES (at V_pad =      *
 * 201088 over 8 shards: T above 2647). The buffer is shared by every call    *
 * on one GPU: calls that overlap on one GPU (other streams, other host      *
 * threads) race on it; calls in one stream are ordered and safe.            *
 * ------------------------------------------------------------------------ */
#define VCE_NOALLOC_SCRATCH_BYTES (16u << 20)
vce_status vce_argmax_noalloc(const void* h, const void* W, int64_t T, int64_t H,
                              int64_t V_real, int64_t V_pad, int32_t num_shards, vce_dtype dt,
                              int32_t* index, float* value, float* shard_value,
                              int32_t* shard_index, void* stream);

/* ------------------------------------------------------------------------ *
 * Explicit (uneven) shard layouts and mapped class ownership.               *
 *                                                                           *
 * [VS] paragraph 1 describes the equal split; [SP] paragraph 5 notes that   *
 * uneven layouts need explicit support. The _ex entry points take the       *
 * layout as shard_rows: a HOST array of num_shards + 1 int64 row offsets,   *
 * 0 first, V_pad last, nondecreasing; shard k owns the physical rows         *
 * [shard_rows[k], shard_rows[k+1]) (an empty shard owns none; V_pad need    *
 * not be a multiple of num_shards). The array is read during the call only. *
 * Everything else (arguments, outputs, rules, errors) is as for the entry   *
 * point without _ex: a shard's maxima/sums and argmax report cover its own  *
 * real rows, an empty shard or one wholly past V_real reports (-inf, 0) and *
 * (-inf, -1). num_shards in [1, 128]; a malformed list gives VCE_ERR_SHARD,  *
 * shard_rows == NULL gives VCE_ERR_NULL. Tiles never cross a shard end.     *
 * The backward does not depend on the layout (every shard's rows receive    *
 * their own gradient rows): call vce_bwd / vemb_bwd with num_shards = 1.    *
 * ------------------------------------------------------------------------ */
size_t vce_fwd_workspace_bytes_ex(int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                                  int32_t num_shards, const int64_t* shard_rows, vce_dtype dt);

vce_status vce_fwd_ex(const void* h, const void* W, const int32_t* targets,
                      int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                      int32_t num_shards, const int64_t* shard_rows, int32_t ignore_index,
                      vce_dtype dt, float* lse, float* loss, float* loss_sum,
                      int32_t* n_valid, int32_t* n_bad_target, float* shard_stats,
                      void* ws, size_t ws_bytes, void* stream);

size_t vce_argmax_workspace_bytes_ex(int64_t T, int64_t H, int64_t V_real, int64_t V_pad,
                                     int32_t num_shards, const int64_t* shard_rows,
                                     vce_dtype dt);

vce_status vce_argmax_ex(const void* h, const void* W, int64_t T, int64_t H, int64_t V_real,
                         int64_t V_pad, int32_t num_shards, const int64_t* shard_rows,
                         vce_dtype dt, int32_t* index, float* value, float* shard_value,
                         int32_t* shard_index, void* ws, size_t ws_bytes, void* stream);

vce_status vemb_fwd_ex(const int32_t* ids, const void* W, int64_t T, int64_t H,
                       int64_t V_real, int64_t V_pad, int32_t num_shards,
                       const int64_t* shard_rows, vce_dtype dt, void* out,
                       int32_t* n_bad_id, void* stream);

/* Mapped ownership: when classes are placed on physical rows by a           *
 * permutation (class c stored at row map[c], map a permutation of           *
 * [0, V_real), the table kept in physical order), IDs and targets are       *
 * translated once before the lookups and the loss:                          *
 *   out[t] = map[in[t]] for in[t] in [0, V_real), else in[t] unchanged      *
 * (so ignore_index and invalid values keep their meaning). The results by   *
 * class are then those of the unmapped table; an argmax index is a physical *
 * row (its class is the inverse map's entry). in and out may be the same    *
 * array. In: in [T], map [V_real] int32.  Out: out [T] int32.               */
vce_status vce_remap(const int32_t* in, int64_t T, const int32_t* map, int64_t V_real,
                     int32_t* out, void* stream);

/* ------------------------------------------------------------------------ *
 * Sampled-softmax candidates.                                               *
 *                                                                           *
 * [SS] Setup (the simplified loss): candidates are the unique targets of    *
 * the batch followed by random negatives, P in all, and each token's        *
 * cross-entropy target is its target's position among the candidates.      *
 * U = the distinct targets in [0, V), ascending. The negatives are the first *
 * P - |U| entries of perm (a caller-drawn random permutation of [0, V)) that *
 * are not in U, so they are uniform without replacement over the rest of    *
 * the vocabulary. cand = U followed by the negatives; n_cand = max(P, |U|). *
 * pos[t] = index of targets[t] in U for targets in [0, V), else targets[t]  *
 * unchanged (so ignore_index stays ignored, other values stay invalid).     *
 * In:  targets [T], perm [V] int32.  Out: cand [cand_cap] int32 with        *
 *      cand_cap >= max(P, min(T, V)); pos [T] int32; n_unique [1], n_cand   *
 *      [1] int32. The candidate rows' gather and cross-entropy reuse       *
 *      vemb_fwd and vce_fwd/vce_bwd (V_real = V_pad = n_cand, one shard);    *
 *      vss_scatter takes the candidate rows' gradient back to the table.     *
 * Errors: T < 0, V < 1, P < 1, P > V (the candidates are distinct rows),    *
 * ignore_index in [0, V) or cand_cap too small: VCE_ERR_SHAPE; a NULL       *
 * pointer: VCE_ERR_NULL; misaligned: VCE_ERR_ALIGN; workspace too small:    *
 * VCE_ERR_WORKSPACE.                                                        *
 * ------------------------------------------------------------------------ */
size_t vss_candidates_workspace_bytes(int64_t T, int64_t V);

vce_status vss_candidates(const int32_t* targets, int64_t T, int64_t V, int32_t ignore_index,
                          const int32_t* perm, int64_t P, int32_t* cand, int64_t cand_cap,
                          int32_t* pos, int32_t* n_unique, int32_t* n_cand,
                          void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ *
 * Sampled-softmax gradient scatter.                                         *
 *                                                                           *
 * [SS] Setup: only the candidate rows take part in the loss, so only they   *
 * receive gradient. For i < P with cand[i] in [0, V): dW[cand[i]] = dWc[i]  *
 * (accumulate = 0: every other row of dW is set to zero) or dW[cand[i]] +=  *
 * dWc[i] (accumulate = 1); other entries of cand are skipped. The entries   *
 * in [0, V) must be distinct, as vss_candidates makes them (a repeated     *
 * entry leaves its row undefined; vemb_bwd sums IDs that repeat): this is   *
 * vemb_bwd's scatter-add for distinct IDs, without its sort and workspace.  *
 * In:  cand [P] int32, dWc [P, H] f32.  Out: dW [V, H] f32.                 *
 * Errors: P < 0, V < 1 or H <= 0: VCE_ERR_SHAPE; accumulate not 0 or 1:     *
 * VCE_ERR_DTYPE; dW NULL, or cand / dWc NULL with P > 0: VCE_ERR_NULL;      *
 * H % 8 != 0 or a misaligned pointer: VCE_ERR_ALIGN.                        *
 * ------------------------------------------------------------------------ */
vce_status vss_scatter(const int32_t* cand, int64_t P, const float* dWc, int64_t H, int64_t V,
                       float* dW, int32_t accumulate, void* stream);

/* ------------------------------------------------------------------------ *
 * Sampled-softmax gradient scatter into a table kept across steps.          *
 *                                                                           *
 * [SS] Setup: a step's gradient lives in its candidate rows only. A caller  *
 * that keeps one dW table from step to step, zero except at the rows the    *
 * previous call wrote (prev [P_prev]), gets the table that vss_scatter with *
 * accumulate = 0 writes while clearing only those rows: every prev[j] in    *
 * [0, V) is set to zero, then dW[cand[i]] = dWc[i] for cand[i] in [0, V)    *
 * (distinct, as for vss_scatter). P_prev*H*4 bytes are cleared instead of   *
 * V*H*4. Precondition: every row of dW not listed in prev is zero (the      *
 * caller zeroes the table once, before its first call, with P_prev = 0).    *
 * On such a table the result has the same bits as vss_scatter(cand, P, dWc, *
 * H, V, dW, 0). prev may repeat rows, share rows with cand and hold values  *
 * outside [0, V) (skipped). The two steps run in order on the stream.       *
 * In:  prev [P_prev] int32, cand [P] int32, dWc [P, H] f32.                 *
 * Out: dW [V, H] f32.                                                       *
 * Errors: P_prev < 0 or as vss_scatter: VCE_ERR_SHAPE; prev NULL with       *
 * P_prev > 0, or as vss_scatter: VCE_ERR_NULL; misaligned prev, or as       *
 * vss_scatter: VCE_ERR_ALIGN.                                               *
 * ------------------------------------------------------------------------ */
vce_status vss_scatter_replace(const int32_t* prev, int64_t P_prev, const int32_t* cand, int64_t P,
                               const float* dWc, int64_t H, int64_t V, float* dW, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VCE_H */
