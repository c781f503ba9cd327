/*
 * sdm.h - Sparse Delta Memory (SDM) chunked write/read, exact product-key top-k and single-token decode step,
 * as a C ABI over hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The method (sparse-delta-memory README.md, summary; CHANGELOG.md 2.0.0): a sequence mixer that keeps a large bank
 * of slots per head. For every token and head it
 *   1. addresses slots with product keys: the query is split into F factors, each factor is scored against its own
 *      sub-key table, and a slot (one sub-key per factor) scores the float32 sum of its factor scores; the top-k
 *      slots are exact (equal to brute force over all slots); equal slot scores go to the larger rank sum, then the
 *      larger first rank (CHANGELOG 2.0.0, "Upgrading from v1" and "New");
 *   2. applies a gated forget/input delta-rule update to the num_writes selected rows (README summary; gated delta
 *      rule of Gated DeltaNet, README "ideas");
 *   3. reads a score-weighted sum of the num_reads selected rows (CHANGELOG 2.0.0, "Removed": the op gathers its own
 *      rows);
 *   processing chunk_size tokens at a time; chunk_size changes results only through floating-point rounding
 *   (CHANGELOG 2.0.0, "Upgrading from v1"). The decode step is the one-token case with a successor bank that may be
 *   the predecessor's own storage (lumen PR #29, "Donating is a permission, not a demand").
 *
 * Arithmetic, as this library defines it (per stream s = (b, h), per token t, all address work bank-independent):
 *   factor score   s_f[i] = float32( fp64 fused-multiply-add chain over c = 0..dk-1 of q[f*dk + c] * C_f[h][i][c] )
 *   rank order     per factor by (score descending, index ascending); p_f = position (0 = best)
 *   slot           (i_0, ..., i_{F-1}); id = ((i_0 * n_1 + i_1) * n_2 + i_2) ...; score = float32 sum, left to right
 *   top-k order    slot score descending, then sum of p_f ascending, then p_0 ascending, p_1 ascending, ...
 *   weights        w = softmax of the W selected write scores, rho = softmax of the R selected read scores
 *   update         r = sum_i w_i M[S_i];  delta = beta * (v - alpha * r);  M[S_i] <- alpha * M[S_i] + w_i * delta
 *   read           out = sum_i rho_i M[R_i], after the update
 * alpha (forget gate) and beta (input gate) are one scalar each per (token, head), given by the caller.
 *
 * Layouts (row-major; every tensor is dense except the bank, whose rows may be padded to bank_row_stride):
 *   queries / write_keys / read_queries  [B, T, H, F*dk]   act dtype; factor f uses columns [f*dk, (f+1)*dk)
 *   subkeys                              [H, sum_f n_f, dk] act dtype; factor tables stacked in factor order
 *   values, out                          [B, T, H, d]      act dtype
 *   forget_gate, input_gate              [B, T, H]         act dtype
 *   bank                                 [B, H, bank_rows, d] bank dtype, row pitch bank_row_stride elements (padding
 *                                        columns are never read or written); rows >= N are never read or written;
 *                                        [H, bank_rows, d] with cfg.shared_bank (sdm_write_read)
 *   write_idx, read_idx (optional)       [B, T, H, W] / [B, T, H, R] int32 slot ids, best first
 *
 * Ownership and streams: the caller owns every buffer. The library never allocates or frees memory (temporary
 * storage comes from the caller's workspace, sized by sdm_workspace_size), never synchronises the stream, keeps no
 * pointer after a call returns, and writes only the outputs named for each call and the workspace. All work is
 * ordered on `stream` (a hipStream_t; NULL = the null stream) of the current HIP device: it starts after the work
 * enqueued on `stream` before the call and ends before the work enqueued after it (sdm_write_read, and the calls
 * that run it: sdm_write_read_save, the layer's forward, may run part of it on a second stream of the library's
 * own, forked from and joined back to `stream`; see sdm_write_read). Results are
 * bitwise repeatable for fixed inputs and settings (no floating-point atomics).
 *
 * Errors: every check runs on the host before any device work, and a refused call does no work (CHANGELOG 2.0.0,
 * "Behavior changes": refusals are raised at the entry of the op, no fallback paths). On a non-OK status,
 * sdm_last_error() returns a message for the calling thread. The device check (gfx950 only) is memoized per device.
 */
#ifndef SDM_H
#define SDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SDM_OK = 0,
  SDM_ERR_DTYPE = 1,          /* float16 (refused, CHANGELOG 2.0.0 "Behavior changes") or an unknown dtype code */
  SDM_ERR_RANGE = 2,          /* a size outside the supported range (listed per field of sdm_config) */
  SDM_ERR_BANK_TOO_SMALL = 3, /* bank_rows < N (CHANGELOG 2.0.0 "Behavior changes": a too-small cache bank) */
  SDM_ERR_ALIAS = 4,          /* an output overlaps an input or another output (except bank_out == bank_in) */
  SDM_ERR_LAYOUT = 5,         /* misaligned pointer, head_dim not a multiple of the bank's 16-byte lane, or a bank
                                 row stride below head_dim or not a 16-byte multiple */
  SDM_ERR_WORKSPACE = 6,      /* workspace NULL, too small, or not 256-byte aligned */
  SDM_ERR_DEVICE = 7,         /* the current device is not gfx950 (no fallback path) */
  SDM_ERR_HIP = 8,            /* a HIP runtime call failed (launch or device query) */
  SDM_ERR_NULL = 9            /* a required pointer is NULL */
} sdm_status;

typedef enum {
  SDM_F32 = 0,
  SDM_BF16 = 1,
  SDM_F16 = 2,  /* always refused */
  SDM_FP8 = 3,  /* snapshot_dtype only: OCP FP8 E4M3 rows in groups of 16 columns with a power-of-two scale */
  SDM_INT4 = 4  /* snapshot_dtype only: int4 rows in [-7, 7], groups of 16 columns with a power-of-two scale */
} sdm_dtype;

typedef struct {
  int32_t batch;            /* B >= 0 */
  int32_t tokens;           /* T >= 0 (exactly 1 for sdm_decode_step) */
  int32_t heads;            /* H >= 0 */
  int32_t num_factors;      /* F in [1, 4] */
  int32_t factor_widths[4]; /* n_f in [1, 4096]; N = prod n_f < 2^31; entries >= F are ignored */
  int32_t subkey_dim;       /* dk >= 1, F * dk <= 1024 */
  int32_t head_dim;         /* d in [1, 2^20]; multiple of 4 (float32 bank) or 8 (bfloat16 bank) */
  int32_t num_writes;       /* W in [1, min(N, 512)] */
  int32_t num_reads;        /* R in [1, min(N, 512)] */
  int32_t chunk_size;       /* C in [1, 65536] (write/read only). The kernels run chunks of at most 128 tokens and
                               8192 write events (C * W); a larger C runs as equal sub-chunks, its largest divisor
                               within those limits (e.g. 256 with W = 64 as two chunks of 128): the chunk size
                               changes results only through rounding, and calls split at multiples of C still give
                               the bits of one call */
  int32_t act_dtype;        /* sdm_dtype of queries, sub-keys, values, gates and out: F32 or BF16 */
  int32_t bank_dtype;       /* sdm_dtype of the bank: F32 or BF16 */
  int64_t bank_rows;        /* rows per stream in the bank buffer, >= N */
  int64_t bank_row_stride;  /* elements from one bank row to the next (0: head_dim); >= head_dim, 16-byte multiple.
                               Performance note: with a row size that is a multiple of 512 bytes, a dense pitch puts
                               the same column slice of every row in one group of HBM channels, and the chunk loop's
                               row gathers then run about 20 % slower (65,536 slots x 1024 float32 columns: 3.3 ms
                               dense vs 2.6 ms per call). A pitch of head_dim + 128 bytes (an odd multiple of
                               128 bytes past the row) spreads the rows over all channels; the library's bandwidth
                               figures are quoted with it. */
  int32_t shared_bank;      /* sdm_write_read only (0 elsewhere): 1 = the B streams of a head share one bank,
                               bank [H, bank_rows, d], and must address disjoint slots (see sdm_shared_bank_check) */
  int32_t snapshot_dtype;   /* read by sdm_write_read_save, sdm_write_read_backward and sdm_snapshot_bytes only:
                               0 = the backward snapshot in the bank dtype, SDM_BF16 = in bfloat16 (on a float32
                               bank: half the bytes; each row rounded to nearest even; on a bfloat16 bank the same
                               as 0), SDM_FP8 / SDM_INT4 = quantized (float32 banks only; see sdm_snapshot_bytes) */
  int32_t topk_scoring;     /* factor-scoring kernel of the batched top-k (ids and scores are identical for every
                               value; only the speed differs): SDM_SCORING_AUTO (0) = the bf16 matrix-core filter
                               where a factor has >= 512 sub-keys, else the fp64 chain over every sub-key;
                               SDM_SCORING_DIRECT = the fp64 chain everywhere; SDM_SCORING_FILTERED = the filter
                               wherever it applies (bf16 activations, factor widths multiples of 16, subkey_dim a
                               multiple of 32 up to 128, 16-byte aligned queries; not the decode step's top-k) */
  int32_t grad_bank_dtype;  /* read by sdm_write_read_backward and sdm_bank_grad_sum only: the element type of
                               grad_bank. 0 (SDM_F32) = float32 accumulation (CHANGELOG 2.0.0 "Deterministic": the
                               grad_bank_fp32 opt-in); SDM_BF16 = the bank dtype of a bfloat16 bank (that page's
                               default), every update of the adjoint bank rounded to bfloat16 (bfloat16 banks with
                               num_writes, num_reads <= 128 only, else SDM_ERR_RANGE before any work) */
} sdm_config;

enum { SDM_SCORING_AUTO = 0, SDM_SCORING_DIRECT = 1, SDM_SCORING_FILTERED = 2 };

enum { SDM_OP_TOPK = 0, SDM_OP_WRITE_READ = 1, SDM_OP_DECODE = 2, SDM_OP_BACKWARD = 3, SDM_OP_DECODE_STEPS = 4 };

/* Message for the last non-OK status returned on the calling thread ("" if none). Valid until the next call. */
const char* sdm_last_error(void);

/* Workspace bytes needed by `op` for `cfg` (k: the top-k size for SDM_OP_TOPK, ignored otherwise).
 * Validates cfg like the op itself, without the device check. */
sdm_status sdm_workspace_size(const sdm_config* cfg, int32_t op, int32_t k, size_t* bytes);

/* Exact product-key top-k (CHANGELOG 2.0.0, "Upgrading from v1" and "New"; README package layout: exact
 * product-key top-k). For every row (b, t, h) of queries [B, T, H, F*dk] (act dtype) against head h's sub-key
 * tables (subkeys [H, sum n_f, dk], act dtype): the k best slots, best first, as int32 ids idx [B, T, H, k] and
 * float32 slot scores scores [B, T, H, k] (scores may be NULL). k in [1, min(N, 512)]. Uses cfg's batch, tokens,
 * heads, factors, subkey_dim and act_dtype; the other fields are not read. */
sdm_status topk_product_keys(const sdm_config* cfg, const void* queries, const void* subkeys, int32_t k,
                             int32_t* idx, float* scores, void* workspace, size_t workspace_bytes, void* stream);

/* The chunked write/read (CHANGELOG 2.0.0: one chunked write/read op; README summary). For every stream (b, h),
 * tokens in order, chunk_size at a time: top-k write slots of write_keys, top-k read slots of read_queries, the
 * gated delta-rule update of the W write rows with values, forget_gate and input_gate, and the read of the R read
 * rows into out. `bank` [B, H, bank_rows, d] advances in place. write_idx / read_idx, if not NULL, receive the
 * selected slot ids. The result equals the one-token-at-a-time recurrence up to floating-point rounding, for any
 * chunk_size; two calls split at a multiple of chunk_size give the same bits as one call.
 * Streams: when the chunk loop's workgroups (one per stream and column slice: B * H * ceil(head_dim * bank bytes /
 * 64), or / 16 for the narrow loop of short rows) fill at most half of the device's compute units, the call runs
 * as up to 16 pieces of whole chunks, the top-k and plan of each piece on a side stream that the library makes once
 * per device (default priority, kept until the process ends) and the chunk loop of each piece on `stream` after
 * that piece's plan: the bits of calls split at those chunks, with the top-k and plan hidden behind the loop. The
 * side stream waits for `stream` at the call's start and `stream` waits for it before the call returns. Calls from
 * several host threads take turns on the side stream. A call on a capturing stream, and a call with shared_bank
 * (its slot check needs every token's top-k before any plan), run in order on `stream`. */
sdm_status sdm_write_read(const sdm_config* cfg, const void* write_keys, const void* read_queries,
                          const void* values, const void* forget_gate, const void* input_gate, const void* subkeys,
                          void* bank, void* out, int32_t* write_idx, int32_t* read_idx, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Training forward (CHANGELOG 2.0.0: training saves a backward snapshot; "Known limitations": the backward restores
 * the bank in place). sdm_write_read, plus `snapshot` [B, H, T, W, d] in the bank dtype, or bfloat16 with
 * cfg.snapshot_dtype = SDM_BF16 (CHANGELOG 2.0.0, "New": bf16 snapshots on a float32 bank) (dense rows, caller-owned):
 * row (b, h, t, i) receives the row of slot write_idx[b, t, h, i] as it was just before token t's write (i in top-k
 * order, best first). The workspace is sdm_write_read's (SDM_OP_WRITE_READ). Refused (SDM_ERR_RANGE) with
 * shared_bank, or when B * H * T * W reaches 2^31 rows (CHANGELOG 2.0.0, "New": a snapshot of 2^31 rows is refused
 * before any work). A bfloat16 snapshot of a float32 bank needs the held-row loop (chunk a power of two in [8, 128],
 * at most 32 terms per lane group) and num_writes, num_reads <= 128, else SDM_ERR_RANGE before any work; its rows are
 * the float32 rows rounded to nearest even, and out and the bank equal the float32 snapshot's bit for bit. Results
 * equal sdm_write_read's up to rounding. */
sdm_status sdm_write_read_save(const sdm_config* cfg, const void* write_keys, const void* read_queries,
                               const void* values, const void* forget_gate, const void* input_gate,
                               const void* subkeys, void* bank, void* out, void* snapshot, int32_t* write_idx,
                               int32_t* read_idx, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the backward snapshot of cfg (cfg.snapshot_dtype), the size of sdm_write_read_save's `snapshot`. With
 * rows = B * H * T * W snapshot rows of d = head_dim columns:
 *   0 (bank dtype) / SDM_BF16: rows * d elements of the bank dtype / bfloat16, [B, H, T, W, d];
 *   SDM_FP8 / SDM_INT4 (CHANGELOG 2.0.0, "New" and "Behavior changes": fp8 and int4 snapshots; their formats are not
 *   given there, so this library's): each row in groups of 16 columns, each group with a power-of-two scale 2^e, e
 *   the smallest exponent with (the group's largest magnitude) / 2^e <= 448 (fp8) or <= 7 (int4); an element x is
 *   stored as the nearest value to x / 2^e, ties to even, of OCP FP8 E4M3 (one byte) or int4 in [-7, 7] (two's
 *   complement nibbles, two per byte, the even column in the low nibble); the buffer holds all elements
 *   [B, H, T, W, d] (rows * d or rows * d / 2 bytes) followed by all scale bytes e + 127 [B, H, T, W, d / 16].
 *   The backward reads the rows back as value times scale (and restores the bank's written rows as those values).
 *   Refused (SDM_ERR_RANGE, before any work), as the pages refuse them: head_dim above 16384, not a multiple of 4, or
 *   not splitting into ceil(head_dim / 128) equal column slices of 16-byte rows; int4 when those slices are 4 mod 8
 *   columns wide; and where this library has no route: a bfloat16 bank, head_dim not a multiple of 16, or settings
 *   outside the held-row loop and the fast reverse sweep (as for SDM_BF16). */
sdm_status sdm_snapshot_bytes(const sdm_config* cfg, size_t* bytes);

/* Deterministic backward of the write/read (CHANGELOG 2.0.0, "Deterministic": every gradient bitwise repeatable;
 * "New": exact product-key top-k with a deterministic sparse backward; "Known limitations": the first backward
 * restores the bank in place). Inputs are the forward's (same cfg, keys, queries, values, gates, sub-keys), `bank`
 * as the forward left it, the forward's `snapshot` (same cfg.snapshot_dtype), and grad_out [B, T, H, d] (act dtype).
 * On return `bank` is the bank before the forward, bit for bit; with a bfloat16 snapshot of a float32 bank, the rows
 * the forward wrote come back rounded to bfloat16 (restored from the snapshot), and every row the backward reads
 * from the snapshot or the restored bank is the rounded one (it enters the key, query, gate and sub-key gradients,
 * not grad_values or grad_bank). grad_bank ([B, H, bank_rows, bank_row_stride], the bank's row layout; float32, or
 * bfloat16 with cfg.grad_bank_dtype = SDM_BF16) holds the gradient w.r.t. the bank after the forward on entry (zeros
 * if none) and the gradient w.r.t. the bank before it on return; in bfloat16 every token's update of a row (its read,
 * then its write) is rounded to nearest even as it is stored. Written (float32, overwritten): grad_write_keys, grad_read_queries [B, T, H, F*dk],
 * grad_values [B, T, H, d], grad_forget_gate, grad_input_gate [B, T, H], grad_subkeys [H, sum n_f, dk] (summed over
 * the batch). The selection itself has no gradient; the gradient reaches keys, queries and sub-keys through the
 * softmax weights of the selected slots, whose scores are sums of factor scores. Workspace: SDM_OP_BACKWARD. The
 * bank and the snapshot are consumed: a second backward of the same forward needs the forward run again. */
sdm_status sdm_write_read_backward(const sdm_config* cfg, const void* write_keys, const void* read_queries,
                                   const void* values, const void* forget_gate, const void* input_gate,
                                   const void* subkeys, void* bank, const void* snapshot, const void* grad_out,
                                   void* grad_bank, float* grad_write_keys, float* grad_read_queries,
                                   float* grad_values, float* grad_forget_gate, float* grad_input_gate,
                                   float* grad_subkeys, void* workspace, size_t workspace_bytes, void* stream);

/* Shared bank (CHANGELOG 2.0.0, "Behavior changes": a direct write/read call that runs several streams over one
 * shared bank must say so, which asserts that the streams' slots are disjoint). With cfg.shared_bank = 1,
 * sdm_write_read takes bank [H, bank_rows, d]: the streams (0, h) ... (B-1, h) all advance bank h. Reading taken
 * here: the streams' slots are disjoint when no slot addressed (written or read) in this call by stream (b, h) is
 * addressed by another stream (b', h); then the streams touch disjoint rows and the result equals running them one
 * after the other. The call checks this on the device after the top-k; if it fails, the call writes neither the
 * bank nor out (the ids may be written) and records the conflict in the workspace. sdm_shared_bank_check waits for
 * `stream` (it synchronises) and sets *conflict to 1 if the last shared-bank sdm_write_read that used this
 * workspace on this stream found a conflict, else 0. cfg and the workspace must be those of that call. */
sdm_status sdm_shared_bank_check(const sdm_config* cfg, const void* workspace, size_t workspace_bytes,
                                 int32_t* conflict, void* stream);

/* Single-token decode step (CHANGELOG 2.0.0 "New": a single-token decode kernel; lumen PR #29: donate). cfg.tokens
 * must be 1; every stream (b, h) takes one token. bank_out == bank_in: donated, the successor is written in place.
 * bank_out disjoint from bank_in: copied successor, bank_out receives a full copy of bank_in with the W rows
 * updated (the whole buffer, B * H * bank_rows * bank_row_stride elements, is copied), and bank_in is left unchanged. Partial overlap -> SDM_ERR_ALIAS. Both forms run one body and give
 * bit-identical bank_out, out and indices. Rows are rounded to the bank dtype before the read. */
sdm_status sdm_decode_step(const sdm_config* cfg, const void* write_keys, const void* read_queries,
                           const void* values, const void* forget_gate, const void* input_gate, const void* subkeys,
                           const void* bank_in, void* bank_out, void* out, int32_t* write_idx, int32_t* read_idx,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Consecutive decode steps in one call (CHANGELOG 2.0.0 "New": a single-token decode kernel; README "CUDA graphs":
 * decode steps replayed without host work in between). cfg.tokens = K >= 0 steps; every input is [B, K, H, ...]
 * (token k of stream (b, h) is step k's input), out [B, K, H, d], write_idx / read_idx (optional) [B, K, H, W|R].
 * The result equals K calls of sdm_decode_step on the tokens in order, bit for bit: the same out rows, ids and
 * final bank (bank_out == bank_in: every step in place; a disjoint bank_out: it receives bank_in's copy once, then
 * every step runs on it, bank_in unchanged). The steps' top-k reads no bank, so all K run first, in parallel; then
 * one launch runs each stream's K steps in order. Shapes: those of sdm_decode_step's one-launch step (num_writes,
 * num_reads <= 64, <= 256 sub-keys per factor, <= 1024 candidate tuples, F * subkey_dim elements a 16-byte multiple,
 * queries and sub-keys 16-byte aligned); others are refused with SDM_ERR_RANGE before any work. Workspace:
 * SDM_OP_DECODE_STEPS with this cfg. */
sdm_status sdm_decode_steps(const sdm_config* cfg, const void* write_keys, const void* read_queries,
                            const void* values, const void* forget_gate, const void* input_gate, const void* subkeys,
                            const void* bank_in, void* bank_out, void* out, int32_t* write_idx, int32_t* read_idx,
                            void* workspace, size_t workspace_bytes, void* stream);

/* The decode step without a workspace, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). Same arguments, checks, kernels and results as
 * sdm_decode_step (bit for bit), except that the temporary storage sdm_decode_step takes from `workspace` comes from
 * a fixed array in device memory that the library holds on each GPU it runs on until the process ends
 * (SDM_NOALLOC_SCRATCH_BYTES per GPU; its address is looked up once per device on the first call there). The call
 * allocates nothing. A step whose workspace (sdm_workspace_size, SDM_OP_DECODE) exceeds SDM_NOALLOC_SCRATCH_BYTES is
 * refused with SDM_ERR_RANGE before any work. Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (other streams or host threads) race and must be serialised by the caller; calls ordered on one
 * stream are safe. */
#define SDM_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
sdm_status sdm_decode_step_noalloc(const sdm_config* cfg, const void* write_keys, const void* read_queries,
                                   const void* values, const void* forget_gate, const void* input_gate,
                                   const void* subkeys, const void* bank_in, void* bank_out, void* out,
                                   int32_t* write_idx, int32_t* read_idx, void* stream);

/* The layer around the op (README usage example: SparseDeltaMemoryArgs(dim, num_heads, slots_per_head, num_writes,
 * num_reads, chunk_size); CHANGELOG 2.0.0, "Behavior changes": a layer call runs the projections, the top-k and the
 * bank copy, then the op; README "ideas": gates of Gated DeltaNet with FLA's A/dt parameterisation). Forward only.
 * With M = B * T rows, Dm = model_dim, P = F * dk and cfg.op the write/read settings:
 *   [keys | queries | values | a | b] = x w_in^T          x [B, T, Dm], w_in [2 H P + H d + 2 H, Dm]: rows
 *                                                         [0, H P) write keys (head-major, [H, P] per token), then
 *                                                         H P read queries, H d values, H forget inputs a, H input
 *                                                         inputs b
 *   alpha = exp(-exp(a_log[h]) * softplus(a + dt_bias[h])),  beta = sigmoid(b)       (float32, rounded to bf16)
 *   o = the write/read op (sdm_write_read) on keys, queries, values, alpha, beta, subkeys and bank
 *   y = o w_out^T                                         o [B, T, H d], w_out [Dm, H d], y [B, T, Dm]
 * Dense maps accumulate in float32 on the matrix cores and round to bfloat16. x, w_in, w_out, subkeys and y are
 * bfloat16 (cfg.op.act_dtype must be SDM_BF16, else SDM_ERR_DTYPE); a_log and dt_bias are float32 [H]. The bank
 * advances in place like sdm_write_read's (shared_bank not allowed). Dm and H * d must be multiples of 32 (the
 * matrix-core step), Dm <= 65536, and every buffer 16-byte aligned (SDM_ERR_RANGE / SDM_ERR_LAYOUT). write_idx /
 * read_idx as in sdm_write_read. The workspace (sdm_layer_workspace_size) holds, in this order and each region
 * starting at a 256-byte multiple: keys [B, T, H, P], queries [B, T, H, P], values [B, T, H, d], gate inputs
 * [B, T, 2 H] (a then b), alpha [B, T, H], beta [B, T, H], o [B, T, H, d] (all bfloat16; left there by the call),
 * then the op's own workspace.
 * Learned initial bank (README model wiring: the bank is learned when backprop_on_memory=true; "Behavior changes":
 * the layer's bank copy runs before the op): initial_bank NULL leaves `bank` the caller's state, advanced in place;
 * initial_bank [H, bank_rows, d] (the bank dtype and row stride) is first copied into the N slot rows of every
 * batch row of `bank` (the per-sequence copy), which the op then advances. Its gradient is the sum over the batch
 * of the op's bank gradient (sdm_bank_grad_sum). */
typedef struct {
  sdm_config op;      /* write/read settings of the op inside the layer */
  int32_t model_dim;  /* Dm, the width of x and y */
  int32_t reserved;   /* 0 */
} sdm_layer_config;

sdm_status sdm_layer_workspace_size(const sdm_layer_config* cfg, size_t* bytes);
sdm_status sdm_layer_forward(const sdm_layer_config* cfg, const void* x, const void* w_in, const float* a_log,
                             const float* dt_bias, const void* w_out, const void* subkeys, const void* initial_bank,
                             void* bank, void* y, int32_t* write_idx, int32_t* read_idx, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Training forward of the layer (CHANGELOG 2.0.0: training saves a backward snapshot): sdm_layer_forward with the
 * op run as sdm_write_read_save (cfg.op.snapshot_dtype; `snapshot` of sdm_snapshot_bytes(&cfg.op)). The workspace
 * must be sdm_layer_backward_workspace_size bytes: its first part is the forward's (same layout), and
 * sdm_layer_backward reads the activations the call leaves there, so it must be passed to the backward untouched. */
sdm_status sdm_layer_forward_save(const sdm_layer_config* cfg, const void* x, const void* w_in, const float* a_log,
                                  const float* dt_bias, const void* w_out, const void* subkeys,
                                  const void* initial_bank, void* bank, void* y, void* snapshot, int32_t* write_idx,
                                  int32_t* read_idx, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of sdm_layer_forward_save and sdm_layer_backward. */
sdm_status sdm_layer_backward_workspace_size(const sdm_layer_config* cfg, size_t* bytes);

/* Backward of the layer (the chain rule through sdm_layer_forward's steps, last first; README model wiring: the layer
 * is trained end to end). Inputs: the forward's x, w_in, a_log, dt_bias, w_out, subkeys, `bank` as the forward left
 * it (the op's backward steps it back to the bank the op started from, as sdm_write_read_backward), its snapshot,
 * grad_y [B, T, Dm] bfloat16 (the gradient w.r.t. y), and the workspace of the sdm_layer_forward_save call.
 * Every tensor between the steps being bfloat16, the gradients passed between them are rounded to bfloat16 too:
 *   d o = grad_y w_out (bfloat16, [B, T, H d])              d w_out = grad_y^T o       (grad_w_out [Dm, H d])
 *   the op's backward on d o (sdm_write_read_backward; grad_bank as there, in and out, cfg.op.grad_bank_dtype)
 *   d a = d alpha alpha (-exp(a_log)) sigmoid(a + dt_bias),  d b = d beta beta (1 - beta)   (float32; alpha and
 *     beta recomputed from the bfloat16 gate inputs), grad_a_log[h] = sum of d alpha alpha (-exp(a_log) softplus),
 *     grad_dt_bias[h] = sum of d a (over every token row, a fixed order)
 *   d p = [d keys | d queries | d values | d a | d b] rounded to bfloat16 ([B, T, N_in], the input map's layout)
 *   d x = d p w_in (grad_x [B, T, Dm])                      d w_in = d p^T x           (grad_w_in [N_in, Dm])
 * grad_subkeys [H, sum n_f, dk] is the op's. Every gradient output is float32 and overwritten (grad_bank excepted).
 * Dense maps accumulate in float32 on the matrix cores. A learned initial bank's gradient is sdm_bank_grad_sum of
 * grad_bank. Workspace regions after the forward's (each at a 256-byte multiple, in this order): the op's region
 * (large enough for its backward), d o [B, T, H d] bfloat16, the op's gradients d keys, d queries [B, T, H P],
 * d values [B, T, H d], d alpha, d beta [B, T, H] (float32), d p [B, T, Np] bfloat16 (Np: N_in rounded up to 64,
 * zero columns past N_in), then scratch. */
sdm_status sdm_layer_backward(const sdm_layer_config* cfg, const void* x, const void* w_in, const float* a_log,
                              const float* dt_bias, const void* w_out, const void* subkeys, void* bank,
                              const void* snapshot, const void* grad_y, void* grad_bank, float* grad_x,
                              float* grad_w_in, float* grad_a_log, float* grad_dt_bias, float* grad_w_out,
                              float* grad_subkeys, void* workspace, size_t workspace_bytes, void* stream);

/* Gradient of a learned initial bank copied into every batch row (sdm_layer_forward's initial_bank): grad_initial_bank
 * [H, bank_rows, bank_row_stride] float32 receives, for every head h, slot j < N and column c < head_dim, the sum over
 * b = 0, 1, ..., B - 1 (in that order, float32) of grad_bank[b, h, j, c] (grad_bank: sdm_write_read_backward's
 * gradient with respect to the bank before the call, [B, H, bank_rows, bank_row_stride], float32 or, with
 * cfg.grad_bank_dtype = SDM_BF16, bfloat16). Rows >= N and padding columns are not written. cfg: the write/read's
 * (per-stream banks). */
sdm_status sdm_bank_grad_sum(const sdm_config* cfg, const void* grad_bank, float* grad_initial_bank, void* stream);

/* Kernel timing (diagnostics, not part of the method). While enabled, every kernel launch of this library is
 * bracketed by a pair of HIP events recorded on the stream it runs on. sdm_profile_read waits for the recorded events
 * and returns, per kernel family, the summed milliseconds (ms) and the number of launches (launches) since timing
 * was enabled; both arrays have SDM_K_COUNT entries and are owned by the caller. Enabling resets the totals;
 * disabling drops pending events. Not thread-safe with concurrent calls on other threads. */
typedef enum {
  SDM_K_CAND = 0,   /* candidate-tuple table */
  SDM_K_TOPK = 1,   /* batched exact top-k */
  SDM_K_PLAN = 2,   /* chunk plan */
  SDM_K_LOOP = 3,   /* chunk loop: gather, solve, read, scatter */
  SDM_K_DECODE = 4, /* decode step */
  SDM_K_COPY = 5,   /* successor copy */
  SDM_K_BWD = 6,    /* backward: reverse sweep, token sums, sub-key sums */
  SDM_K_DENSE = 7,  /* layer: dense maps (projections, output projection) and gates */
  SDM_K_COUNT = 8
} sdm_kernel;
sdm_status sdm_profile_enable(int32_t on);
sdm_status sdm_profile_read(double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* SDM_H */
