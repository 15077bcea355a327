/*
 * lkv.h -- C ABI of the MI355X (gfx950) quantised KV-cache decode library.
 *
 * The three calls follow the pages' statement of the problem:
 *   lkv_quant_append  quantise new K/V rows and bit-pack them into the cache
 *   lkv_decode_attn   attention of the current decode queries against the
 *                     packed cache (split over the token axis, then merged)
 *   lkv_decode_attn_multi  the same for several query tokens per sequence,
 *                     with a causal mask
 *   lkv_tier_update   attention-aware tiers: HIGH keeps 6-bit V, MID gets
 *                     4-bit V, LOW is evicted
 *   lkv_retier        the same tiers applied again to a tiered cache as its
 *                     scores change
 * Sources of each operation are cited at its declaration.
 *
 * Conventions for every call:
 *  - Pointers are device pointers unless marked (host).  The caller owns every
 *    buffer (pools, tables, lengths, Q, K, V, scores, outputs, workspaces);
 *    the library allocates nothing and holds no global state besides its
 *    loaded kernels.
 *  - `stream` is a hipStream_t (0 = the null stream).  Work is queued on it and
 *    never synchronised by the library; device faults surface at the caller's
 *    next synchronisation.
 *  - Host-side argument checks run before any launch: a call that fails them
 *    returns LKV_EINVAL or LKV_EUNSUPPORTED and queues nothing.  A launch
 *    failure reported by the HIP runtime returns LKV_EHIP.
 *  - Calls are thread-safe as long as concurrent calls write distinct buffers.
 *
 * Cache format (one layout for every call).  Tokens are grouped in blocks of
 * 64.  A pool is [num_blocks][num_kv_heads][chunk_bytes]; one chunk holds one
 * block of one KV head in six sections, each padded to a multiple of 128 B:
 *   K codes   64 token rows, each the head_dim channel codes as a k_bits-bit
 *             bitstream
 *   V codes   head_dim channel rows, each the 64 slot codes as a v_bits-bit
 *             bitstream
 *   K scales  fp32 [head_dim/group_size][64]
 *   V scales  fp32 [head_dim/group_size][64]
 *   K zeros   uint8 [head_dim/group_size][64]
 *   V zeros   uint8 [head_dim/group_size][64]
 * A bitstream holds field i in bits [i*b, i*b+b), LSB first, in little-endian
 * 32-bit words.  Element x of channel d in group d/group_size is stored as the
 * code q with scale s and zero point z such that x ~ (q - z) * s.  With
 * k_bits = v_bits = 16 (precision-sensitive layers) the fields are fp16 bit
 * patterns (round to nearest even) and the metadata sections are empty.
 * Logical block i of sequence b lives in pool block block_table[b][i]; a
 * contiguous cache is the identity table.
 *
 * Direction-preserving K (k_norm = 1; the norm-direction page's insight that
 * a key's direction matters more to attention than its norm): quantised
 * formats only.  A seventh section, fp32 [64] (256 B) after the six, holds
 * one factor per slot, r = |k| / |k_hat| (norms in fp64, r rounded to fp32;
 * 1 for a zero k_hat), and every call reads the key as r * k_hat: the
 * direction of the group codes with the norm of the original key.  The
 * codes, scales and zeros are those of the plain format.  lkv_quant_append
 * needs K and V aligned to head_dim / 64 elements for it.  Decode reads the
 * factors in the matrix-core kernels (bf16 Q, head_dim 128, group 64, K6 with
 * V4 or V6, 4 or 8 query heads per KV head, a 16-byte aligned Q, splits of at
 * most 4096 tokens) and in the generic kernel otherwise; the tier calls
 * return LKV_EUNSUPPORTED.
 */
#ifndef LKV_H
#define LKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LKV_BLOCK_TOKENS 64

typedef enum {
    LKV_OK = 0,
    LKV_EINVAL = -1,       /* null pointer, bad size or inconsistent arguments */
    LKV_EUNSUPPORTED = -2, /* a format or shape the library has no kernel for */
    LKV_EHIP = -3,         /* the HIP runtime refused a launch */
    LKV_ESCRATCH = -4      /* lkv_decode_attn_noalloc: the call's partials exceed
                              LKV_NOALLOC_SCRATCH_BYTES */
} lkv_status;

typedef enum { LKV_F32 = 0, LKV_BF16 = 1, LKV_F16 = 2 } lkv_dtype;

/* One cache.  head_dim 64 or 128; group_size 16, 32 or 64 dividing head_dim;
 * (k_bits, v_bits) in {4, 6} x {4, 6}, or (16, 16); block_tokens 64.  pool is
 * 256-byte aligned and holds num_blocks * num_kv_heads * chunk bytes, where
 * chunk is lkv_chunk_layout's off[6], plus 256 when k_norm is 1. */
typedef struct lkv_cache {
    int32_t head_dim;
    int32_t group_size;
    int32_t k_bits;
    int32_t v_bits;
    int32_t num_kv_heads;
    int32_t block_tokens;
    int64_t num_blocks;
    void* pool;
    int32_t k_norm;  /* 1: direction-preserving K (see below); 0: plain */
} lkv_cache;

/* What a batch reads from one cache. */
typedef struct lkv_view {
    const int32_t* block_table; /* [batch][max_blocks] int32 */
    const int32_t* seq_lens;    /* [batch] int32, live tokens per sequence */
    int32_t max_blocks;
    int32_t max_len;            /* (host) upper bound of seq_lens, sizes the grid; a
                                   length above it is out of contract and is read
                                   as max_len */
    int64_t sum_len;            /* (host) hint: total of seq_lens over the batch,
                                   or 0 if unknown; lkv_decode_plan sizes splits
                                   for ragged batches by it, and the merge of a
                                   one-segment call whose sum_len is below
                                   batch * max_len reads only the splits that
                                   hold tokens (the result is the same) */
} lkv_view;

/* Human-readable name of a status. */
const char* lkv_status_string(int status);

/* Byte offsets of the six sections of a chunk and, in off[6], the chunk size
 * (the memory layout reorganised for the quantised format: LeanKV page,
 * implementation details); with k_norm = 1 the factor section starts at
 * off[6] and adds 256 bytes.  Returns LKV_OK or LKV_EUNSUPPORTED. */
int lkv_chunk_layout(int32_t head_dim, int32_t group_size, int32_t k_bits, int32_t v_bits,
                     int64_t off[7]);

/* Quantise and append new rows.
 * Group-wise asymmetric integer quantisation with an fp32 scale and an integer
 * zero point per group of group_size channels along head_dim (TurboQuant
 * page, core innovation), at 6 bits for K and 4 bits for V, or fp16 for
 * precision-sensitive layers (Super KV Compression page, first layer).  Per
 * group, in fp32 with no contraction and correctly rounded division:
 *   constant group c: (s, z, q) = (c, 0, 1), (-c, 1, 0) or (0, 0, 0);
 *   otherwise lo = min(min x, 0), hi = max(max x, 0), s = (hi - lo) / qmax,
 *   z = clamp(rint(-lo / s)), q = clamp(rint(x / s) + z), qmax = 2^bits - 1,
 *   rint rounding half to even.
 * k, v       [total_new][num_kv_heads][head_dim] in `dtype` (LKV_F32/BF16/F16)
 * cu_new     [batch+1] int32, rows of sequence b are cu_new[b] .. cu_new[b+1]-1
 * start_pos  [batch] int32, cache position of the first new row of b
 * block_table[batch][max_blocks]; every block the rows land in must be mapped
 * max_new    (host) upper bound of cu_new[b+1]-cu_new[b]; sizes the grid
 * Writes the rows' codes, scales and zeros and nothing else in the pool.
 * Sequence lengths are not updated: the caller advances its seq_lens. */
int lkv_quant_append(const lkv_cache* cache, const void* k, const void* v, int32_t dtype,
                     const int32_t* cu_new, const int32_t* start_pos,
                     const int32_t* block_table, int32_t max_blocks,
                     int32_t batch, int32_t max_new, void* stream);

/* Split plan of lkv_decode_attn: a multiple of 64 tokens per split, chosen
 * from the shapes alone (deterministic).  It aims at about 2048 splits with
 * work: a sequence is counted at max_len tokens, or, when views carry a
 * sum_len hint, the batch at sum_len tokens.  (host) */
int lkv_decode_plan(const lkv_cache* segs, const lkv_view* views, int32_t nseg,
                    int32_t batch, int32_t num_q_heads, int32_t* split_tokens);

/* Split plan of a one-segment decode step (lkv_append_decode,
 * lkv_append_split) for a host that also knows every sequence's length.  A
 * ragged batch (view->sum_len below batch * max_len) of at most 64 sequences
 * in a format with the fused matrix-core step (head_dim 128, K6, V4 or V6,
 * plain K, 4 or 8 query heads per KV head) runs only its splits with tokens,
 * each in its own wave: the smallest split whose count of such splits over
 * the KV heads (an empty sequence counts one) is at most 2048.  Otherwise
 * lkv_decode_plan's choice.  host_lens [batch] int32, host memory: the
 * lengths the call will see (the new token counted).  Lengths that differ
 * from the device's change only the speed.  (host) */
int lkv_decode_plan_lens(const lkv_cache* cache, const lkv_view* view, const int32_t* host_lens,
                         int32_t batch, int32_t num_q_heads, int32_t* split_tokens);

/* Bytes of workspace lkv_decode_attn needs for a split size (host):
 * fp32 partials [batch][num_q_heads][total_splits][head_dim + 2]. */
int64_t lkv_decode_workspace_bytes(const lkv_cache* segs, const lkv_view* views, int32_t nseg,
                                   int32_t batch, int32_t num_q_heads, int32_t split_tokens);

/* Decode attention over the packed cache.
 * For each sequence b and query head h (KV head h / (num_q_heads /
 * num_kv_heads)), softmax(sm_scale * q . k_hat) over every live token of
 * every segment (segments in order; nseg 1, or 2 for a tiered cache {HIGH,
 * MID}), weighted sum of v_hat, where k_hat, v_hat = (q - z) * s.  Tokens are
 * processed per split of split_tokens (0 = lkv_decode_plan's choice),
 * counted from the start of each segment, and per 64-token block inside a
 * split.  Sparse-V skip (Super KV Compression page, third layer): after a
 * block's scores are folded into the split's running maximum m and sum L,
 * the V term of token j for head h is skipped when
 *   exp(s_j - m) < tau_low * L;
 * skipped tokens stay in the softmax denominator.  tau_low <= 0 skips
 * nothing.  Partial results of the splits are merged by a second kernel.
 * q          [batch][num_q_heads][head_dim] in q_dtype (LKV_F32 or LKV_BF16)
 * out        [batch][num_q_heads][head_dim] fp32
 * workspace  lkv_decode_workspace_bytes() bytes, 256-byte aligned
 * The cache is only read. */
int lkv_decode_attn(const lkv_cache* segs, const lkv_view* views, int32_t nseg,
                    const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                    float sm_scale, float tau_low, int32_t split_tokens,
                    float* out, void* workspace, size_t workspace_bytes, void* stream);

/* One decode step of a layer in one call: lkv_quant_append of each
 * sequence's new K and V row, then lkv_decode_attn over the cache that
 * holds it (the pages' two operations in sequence: quantise and pack the new
 * token, TurboQuant page core innovation and Super KV Compression page first
 * layer; then attention over the packed cache, which includes the token
 * appended in the same step).  One segment.
 * view.seq_lens[b] already counts the new token: its row goes to position
 * seq_lens[b] - 1 (through view.block_table, which must map that block) and
 * attention reads seq_lens[b] tokens.  A sequence of length 0 appends
 * nothing and gives a zero row.
 * k_new, v_new  [batch][num_kv_heads][head_dim] in kv_dtype (LKV_F32, BF16
 *               or F16); with k_norm, aligned as lkv_quant_append requires
 * Other arguments, the workspace and out as lkv_decode_attn (split_tokens
 * 0 = lkv_decode_plan()).  The pool and out are exactly those of
 * lkv_quant_append (cu_new = 0, 1, .., batch; start_pos = seq_lens - 1)
 * followed by lkv_decode_attn.  For bf16 Q, head_dim 128, group 64, K6
 * with V4 or V6, 4 or 8 query heads per KV head and new rows aligned to two
 * channels, the split kernel writes the rows itself (the wave whose split
 * holds a sequence's newest token), so the step is two launches; other
 * formats run the append kernel first. */
int lkv_append_decode(const lkv_cache* cache, const lkv_view* view, const void* k_new, const void* v_new,
                      int32_t kv_dtype, const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                      float sm_scale, float tau_low, int32_t split_tokens, float* out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* The decode step of a layer in one launch: the split kernel appends each
 * sequence's new row, as lkv_append_decode does, and also merges the split
 * partials (the combine step of the split decode).  A workgroup of G waves
 * (G = query heads per KV head, 4 or 8) runs G consecutive splits of a
 * (sequence, KV head) and merges them in LDS; the last of a row's
 * workgroups to finish merges the row's workgroup partials into the output.
 * segs, views, nseg: one segment (the formats for which lkv_append_decode
 * writes the new rows in the split kernel), or a tiered cache's two
 * segments (Super KV Compression page, second layer): segs[0] HIGH (K6V6)
 * and segs[1] MID (K6V4), head_dim 128, group 64, bf16 Q, 4 or 8 query
 * heads per KV head, no direction-preserving K.  The new rows go to
 * segs[0] at views[0].seq_lens[b] - 1, as lkv_quant_append would write
 * them; attention reads every segment, with the sparse-V skip at tau_low.
 * One segment whose view marks a ragged batch (sum_len below batch x
 * max_len) of at most 64 sequences runs in the compact order of
 * lkv_append_decode (every wave a split with tokens; lkv_decode_plan_lens
 * sizes the splits), its workgroups merging the runs of consecutive splits
 * they hold.  The pool is exactly that of lkv_quant_append then lkv_decode_attn; the
 * output is the same attention merged in another order (G splits at a
 * time, then the groups), so it may differ from theirs in the last bits.
 * counters: uint32 [batch][number of KV heads], caller-owned, all zero
 * before the first call (a zero-filled allocation); every completed call
 * leaves them zero.  Calls that share counters or a workspace must not
 * overlap.  At most 256 G splits per sequence over all segments; otherwise,
 * or for another format or shape, LKV_EUNSUPPORTED and nothing is launched
 * (lkv_append_decode, or lkv_quant_append then lkv_decode_attn, serves
 * every case).  nseg other than 1 or 2: LKV_EINVAL.  Workspace:
 * lkv_decode_workspace_bytes() of the same segments. */
int lkv_append_decode_merged(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* k_new,
                             const void* v_new, int32_t kv_dtype, const void* q, int32_t q_dtype, int32_t batch,
                             int32_t num_q_heads, float sm_scale, float tau_low, int32_t split_tokens, float* out,
                             uint32_t* counters, void* workspace, size_t workspace_bytes, void* stream);

/* The first stage of lkv_append_decode, for callers that schedule the two
 * apart (lkv_append_decode is exactly lkv_append_split followed by
 * lkv_decode_combine on the same stream): the new rows and the split
 * partials.  split_tokens must be the resolved (non-zero) split size. */
int lkv_append_split(const lkv_cache* cache, const lkv_view* view, const void* k_new, const void* v_new,
                     int32_t kv_dtype, const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                     float sm_scale, float tau_low, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                     void* stream);

/* lkv_decode_attn for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace and allocates nothing: the split
 * partials go to a static device array of LKV_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends.  Same
 * arguments, kernels, split plan and output as lkv_decode_attn.
 * The array is shared by every call on one GPU and keeps the last call's
 * contents (the partials need no initialisation): calls that overlap on one
 * GPU -- on different streams, or from several threads -- race, so the
 * caller orders them.  Returns LKV_ESCRATCH when the call's partials,
 * lkv_decode_workspace_bytes(), exceed LKV_NOALLOC_SCRATCH_BYTES. */
#define LKV_NOALLOC_SCRATCH_BYTES (16u << 20)
int lkv_decode_attn_noalloc(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* q,
                            int32_t q_dtype, int32_t batch, int32_t num_q_heads, float sm_scale, float tau_low,
                            int32_t split_tokens, float* out, void* stream);

/* Measurement helper, not a step of the method: a streaming read of
 * `bytes` of the device buffer buf, the bandwidth a read-only kernel
 * reaches on this part, against which the decode kernels' fractions of the
 * HBM peak are read.  One launch of (compute units x 8) workgroups of 256
 * threads, each thread keeping four 16-byte loads in flight over a
 * grid-stride loop; nontemporal != 0 loads with the non-temporal hint.
 * sink: one device uint32, written only if the buffer's words xor-fold to
 * 0x9E3779B9 (never for a zero-filled buffer).  buf 16-byte aligned, bytes
 * a positive multiple of 16, else LKV_EINVAL. */
int lkv_hbm_read_probe(const void* buf, int64_t bytes, int32_t nontemporal, uint32_t* sink, void* stream);

/* Split size for lkv_decode_attn_multi (host): lkv_decode_plan over the
 * work items the call launches, batch * T query tokens, or batch * ceil(T/2)
 * query-token pairs at 4 query heads per KV head (the matrix-core kernel
 * then runs two tokens of a sequence through one pass over its blocks). */
int lkv_decode_plan_multi(const lkv_cache* segs, const lkv_view* views, int32_t nseg,
                          int32_t batch, int32_t q_per_seq, int32_t num_q_heads, int32_t* split_tokens);

/* Attention of several query tokens per sequence over the packed cache,
 * with a causal mask: the queries of a chunked prefill, or draft tokens to
 * verify.  The TurboQuant page states that the quantised cache stacks with
 * FlashAttention-style attention; this is that computation over it.
 * q_per_seq = T query tokens per sequence; their K and V rows are already
 * appended and are the last T tokens of the first segment (seq_lens count
 * them).  Query token i of sequence b attends to that segment's tokens
 * 0 .. L_b - T + i and to every token of the other segments: each query
 * token is one lkv_decode_attn query over its causal prefix, with the same
 * split size and sparse-V rule.
 * q          [batch][T][num_q_heads][head_dim] in q_dtype
 * out        [batch][T][num_q_heads][head_dim] fp32
 * split_tokens  0 = lkv_decode_plan_multi()
 * workspace  lkv_decode_workspace_bytes(..., batch * T, ...) bytes
 * views[0].max_len must be at least T; a sequence shorter than T gives
 * zero rows for the queries that see no token.  T = 1 is lkv_decode_attn. */
int lkv_decode_attn_multi(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* q,
                          int32_t q_dtype, int32_t batch, int32_t q_per_seq, int32_t num_q_heads, float sm_scale,
                          float tau_low, int32_t split_tokens, float* out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* lkv_decode_attn_multi (q_per_seq = T; 1 is lkv_decode_attn) that also
 * reports every sparse-V skip decision, for tests that compare skip sets
 * bit for bit (Super KV Compression page, third layer: the V term of a
 * token under the threshold is not dequantised).  The rule compares
 * exp(s - m) with tau_low * L in fp32; near the bound a test takes this
 * call's decision as one of the correct ones.  The kernels, split plan and
 * output are those of lkv_decode_attn_multi; only the mask is added.
 * skip_mask  uint32 [batch * q_per_seq][num_q_heads][mask_words]; bit c of
 *            a row (word c / 32, bit c % 32) is set when the V term of score
 *            column c was skipped for that query head.  Column c is token
 *            c of the first segment, or token c - C0 of the second, where
 *            C0 = views[0].max_len rounded up to 64.  Bits of columns
 *            without a live token are 0.  The call clears the mask first.
 * mask_words >= (sum over segments of max_len rounded up to 64) / 32
 * Other arguments as lkv_decode_attn_multi (split_tokens 0 =
 * lkv_decode_plan_multi()).  Not for production use: the skip decisions
 * cost one atomic per skipped pair. */
int lkv_decode_attn_debug(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* q,
                          int32_t q_dtype, int32_t batch, int32_t q_per_seq, int32_t num_q_heads, float sm_scale,
                          float tau_low, int32_t split_tokens, float* out, uint32_t* skip_mask, int32_t mask_words,
                          void* workspace, size_t workspace_bytes, void* stream);

/* The two stages of lkv_decode_attn, for callers that schedule them apart
 * (lkv_decode_attn is exactly lkv_decode_split followed by
 * lkv_decode_combine on the same stream).  split_tokens must be the
 * resolved (non-zero) split size.  lkv_decode_split writes the partial
 * (o[head_dim], m, L) of every split; a split past its sequence's end writes
 * only m = -inf and L = 0, and lkv_decode_combine gives it weight 0 and
 * never uses its o row, so the workspace needs no initialisation. */
int lkv_decode_split(const lkv_cache* segs, const lkv_view* views, int32_t nseg,
                     const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                     float sm_scale, float tau_low, int32_t split_tokens,
                     void* workspace, size_t workspace_bytes, void* stream);
int lkv_decode_combine(const lkv_cache* segs, const lkv_view* views, int32_t nseg,
                       int32_t batch, int32_t num_q_heads, int32_t split_tokens,
                       float* out, const void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of lkv_decode_attn_scores (host): the decode partials,
 * then fp32 score rows [batch][num_q_heads][sum over segments of max_len
 * rounded up to 64], then (M, 1/L) fp32 pairs [batch][num_q_heads], each part
 * 256-byte aligned. */
int64_t lkv_decode_scores_workspace_bytes(const lkv_cache* segs, const lkv_view* views, int32_t nseg,
                                          int32_t batch, int32_t num_q_heads, int32_t split_tokens);

/* lkv_decode_attn that also accumulates attention scores: the per-token
 * signal of the attention-aware tiers (Super KV Compression page, second
 * layer).  For every live token j of segment s of sequence b it adds
 *   score_acc[s][b][j] += sum over query heads h of a_bhj,
 * a_bhj = exp(s_bhj - M_bh) / L_bh, the token's softmax weight for head h
 * over all live tokens of all segments (the weights of skipped tokens
 * included: the skip drops only their V term).  out is exactly what
 * lkv_decode_attn writes.  score_acc: fp32 [nseg][batch][acc_stride],
 * acc_stride >= every view's max_len; entries past a sequence's length are
 * left untouched.  workspace: lkv_decode_scores_workspace_bytes() bytes,
 * 256-byte aligned.  The cache is only read. */
int lkv_decode_attn_scores(const lkv_cache* segs, const lkv_view* views, int32_t nseg,
                           const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                           float sm_scale, float tau_low, int32_t split_tokens, float* out,
                           float* score_acc, int32_t acc_stride, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Thresholds from the quantisation error bound (Super KV Compression page,
 * second layer), for n live tokens (host):
 *   tau_low = eps4 / n,  tau_high = (eps4 / eps6) / n,  eps_b = 1/(2(2^b - 1)).
 * Evicting every token of weight < tau_low moves an output by at most
 * eps4 * max|v|, the 4-bit half-step relative to a group's range. */
void lkv_default_thresholds(int32_t n_tokens, float* tau_low, float* tau_high);

/* Workspace bytes of lkv_tier_update (host): (HIGH, MID) int32 counts per
 * 2048-token scan chunk of each sequence, then the (HIGH, MID) destination
 * positions of every 64-token block of each sequence, then 8 bytes and a
 * uint32 per 64-token block of each sequence for in-place compaction:
 * batch * (ceil(scores_stride / 2048) + ceil(scores_stride / 64)) * 8 + 8
 * + batch * ceil(scores_stride / 64) * 4 bytes (each ceil at least 1).  The
 * workspace must be 8-byte aligned; its contents need no initialisation. */
int64_t lkv_tier_workspace_bytes(int32_t batch, int32_t scores_stride);

/* Attention-aware tier update (Super KV Compression page, second layer).
 * src is a K6/V6 cache.  For token j < seq_len[b] with score s = scores[b][j]:
 *   s >= tau_high             HIGH: K6 row and V6 row copied bit for bit into
 *                             dst_h (K6/V6)
 *   tau_low <= s < tau_high   MID: K6 row copied, V dequantised in fp32
 *                             ((q - z) * s) and requantised at 4 bits into
 *                             dst_m (K6/V4)
 *   s < tau_low               LOW: evicted
 * Survivors are written from position 0 of their destination in increasing
 * token order (block tables h_block_table, m_block_table).  tiers[b][j]
 * receives 2, 1 or 0 for j < seq_len[b]; n_high[b], n_mid[b] the counts.  If
 * a destination has fewer than the count's slots (max_blocks * 64), the
 * count is returned negated and nothing is written to either destination for
 * that sequence.  scores, tiers: [batch][scores_stride]; workspace:
 * lkv_tier_workspace_bytes() bytes.  src is only read, unless dst_h is src
 * compacted in place: the same pool and the same block table (pointer and
 * h_max_blocks equal to the view's max_blocks).  Then the HIGH tokens end
 * at positions 0 .. n_high-1 of src's own blocks, the blocks of a row past
 * ceil(n_high / 64) hold no live token and may be reused, and the slots past
 * n_high keep stale codes.  Otherwise no destination block may be one src
 * uses; dst_m with src's pool and block table is LKV_EINVAL. */
int lkv_tier_update(const lkv_cache* src, const lkv_view* src_view,
                    const float* scores, int32_t scores_stride, float tau_low, float tau_high,
                    const lkv_cache* dst_h, const int32_t* h_block_table, int32_t h_max_blocks,
                    const lkv_cache* dst_m, const int32_t* m_block_table, int32_t m_max_blocks,
                    int32_t* n_high, int32_t* n_mid, uint8_t* tiers, int32_t batch,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of lkv_retier (host): the (HIGH, MID) int32 counts of
 * every 2048-token scan chunk and the (HIGH, MID) destination positions of
 * every 64-token block, of both segments, then the in-place compaction's
 * 8 bytes and uint32 per 64-token block of the longer segment:
 * batch * (ceil(h_stride / 2048) + ceil(m_stride / 2048) + ceil(h_stride / 64)
 * + ceil(m_stride / 64)) * 8 + 8 + batch * max(ceil(h_stride / 64),
 * ceil(m_stride / 64)) * 4 bytes (each ceil at least 1).  8-byte aligned;
 * its contents need no initialisation. */
int64_t lkv_retier_workspace_bytes(int32_t batch, int32_t h_stride, int32_t m_stride);

/* Re-tiering of a tiered cache with fresh scores (the attention-aware tiers
 * applied again as the scores change, Super KV Compression page, second
 * layer).  h is the HIGH segment (K6/V6 or K4/V6), m the MID segment (same K,
 * V4), each with its view and its scores ([batch][h_stride],
 * [batch][m_stride], fp32).  For a HIGH token with score s:
 *   s >= tau_high             stays HIGH: copied bit for bit into dst_h
 *   tau_low <= s < tau_high   demoted to MID: K copied, V dequantised in fp32
 *                             and requantised at 4 bits into dst_m
 *   s < tau_low               evicted
 * and for a MID token: s >= tau_low stays MID (copied bit for bit into dst_m;
 * its 6-bit V is gone, so a MID token is never promoted), else evicted.
 * dst_h receives the kept HIGH tokens in token order; dst_m the kept MID
 * tokens in token order, then the demoted tokens in token order, each from
 * position 0 (block tables dh_block_table, dm_block_table).  h_tiers[b][j]
 * and m_tiers[b][j] receive each live token's new tier (2, 1 or 0); n_high
 * and n_mid the new lengths.  If a destination has fewer than the count's
 * slots, both counts are returned negated and nothing is written to either
 * destination for that sequence.  n_high, n_mid must not be the sources'
 * seq_lens.  Workspace: lkv_retier_workspace_bytes().
 *
 * In place: dst_h may be h and dst_m may be m, each the same pool and the
 * same block table (pointer and max_blocks equal to its view's), so that a
 * re-tier needs no second set of blocks.  A segment is then compacted
 * within its own blocks (MID first, then HIGH, one launch after the other;
 * within a segment a token never moves to a later position).  The MID row
 * must hold valid blocks for n_mid positions, at most m_len + h_len: the
 * demoted tokens follow the kept MID ones.  Afterwards the blocks of a row
 * past ceil(n / 64) hold no live token and may go back to a free list; the
 * slots past n keep stale codes.  Any other
 * overlap between destination blocks and the blocks a source uses is not
 * allowed; dst_h with m's pool and block table, or dst_m with h's, is
 * LKV_EINVAL.  (A block table shared between different pools names
 * different blocks and is no overlap.) */
int lkv_retier(const lkv_cache* h, const lkv_view* h_view, const float* h_scores, int32_t h_stride,
               const lkv_cache* m, const lkv_view* m_view, const float* m_scores, int32_t m_stride,
               float tau_low, float tau_high,
               const lkv_cache* dst_h, const int32_t* dh_block_table, int32_t dh_max_blocks,
               const lkv_cache* dst_m, const int32_t* dm_block_table, int32_t dm_max_blocks,
               int32_t* n_high, int32_t* n_mid, uint8_t* h_tiers, uint8_t* m_tiers, int32_t batch,
               void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LKV_H */
