/*
 * lkv_oracle.h -- plain CPU oracle for the quantised KV-cache decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes this
 * header or links this code; only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares no source with the HIP
 * library (which has its own header, include/lkv.h).
 *
 * What it computes, and where that comes from:
 *  - group-wise asymmetric integer quantisation with a scale and a zero point
 *    ("TurboQuant" page, section on the core innovation: asymmetric and
 *    grouped quantisation with a scale computation);
 *  - 6-bit keys, 4-bit values, fp16 for precision-sensitive layers
 *    ("Super KV Compression" page, first layer);
 *  - a memory layout reorganised for the quantised format ("LeanKV" page,
 *    implementation details);
 *  - softmax attention of one decode query over the dequantised cache;
 *  - attention-aware tiers (high keeps 6-bit V, mid 4-bit V, low evicted)
 *    with thresholds from the quantisation error bound ("Super KV
 *    Compression" page, second layer);
 *  - skipping V dequantisation for low-weight tokens (same page, third layer).
 *
 * Precision: quantisation is fp32 with a fixed operation order, no FMA
 * contraction (build with -ffp-contract=off), correctly rounded division and
 * ties-to-even rounding.  Attention is fp64.
 */
#ifndef LKV_ORACLE_H
#define LKV_ORACLE_H
#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_BLOCK_TOKENS 64

/* One cache ("segment"): format plus a host pool [num_blocks][Hkv][chunk]. */
typedef struct orc_cache {
    int32_t head_dim;      /* D */
    int32_t group_size;    /* g, channels per quantisation group */
    int32_t k_bits;        /* 4, 6 or 16 (16 = fp16 passthrough) */
    int32_t v_bits;        /* 4, 6 or 16; 16 only together with k_bits 16 */
    int32_t num_kv_heads;  /* Hkv */
    int64_t num_blocks;
    uint8_t* pool;
    int32_t k_norm;        /* 1: direction-preserving K (a per-token norm factor
                              after the six sections); quantised formats only */
} orc_cache;

/* Which blocks of a cache a batch reads: host block table and lengths. */
typedef struct orc_view {
    const int32_t* block_table; /* [batch][max_blocks] */
    const int32_t* seq_lens;    /* [batch] */
    int32_t max_blocks;
} orc_view;

/* Section offsets of one chunk: K codes, V codes, K scales, V scales,
 * K zeros, V zeros, and [6] = chunk bytes.  Returns 0, or -1 if the format
 * is not one the method defines. */
int orc_chunk_layout(int D, int g, int kb, int vb, int64_t off[7]);

/* Quantise one group of n fp32 values at `bits` (4 or 6). */
void orc_quantize_group(const float* x, int n, int bits,
                        float* scale, uint8_t* zero, uint8_t* codes);

/* Bitstream helpers: field idx of width `bits`, LSB first. */
uint32_t orc_get_field(const uint8_t* stream, int64_t idx, int bits);
void orc_put_field(uint8_t* stream, int64_t idx, int bits, uint32_t value);

/* fp32 -> fp16 bit pattern, round to nearest even, subnormals kept. */
uint16_t orc_f32_to_f16(float x);
double orc_f16_to_f64(uint16_t h);

/* Quantise-and-append rows.  k, v: fp32 [total_new][Hkv][D] (inputs of
 * narrower dtypes are widened exactly by the caller).  cu_new [batch+1],
 * start_pos [batch], block_table [batch][max_blocks]. */
int orc_append(const orc_cache* c, const float* k, const float* v,
               const int32_t* cu_new, const int32_t* start_pos,
               const int32_t* block_table, int32_t max_blocks, int32_t batch);

/* Decode attention (fp64).  q: fp32 [batch][Hq][D].  Segments are read in
 * order; split_tokens is a multiple of 64 (0 = one split per segment).
 * tau_low <= 0 disables the sparse-V skip.  out: fp64 [batch][Hq][D].
 * skip (optional, may be NULL): uint8 [batch][Hq][nseg][max_tok] where
 * max_tok = max over segments of max_blocks*64; 1 = V term skipped.
 * score_acc (optional, may be NULL): fp64 [nseg][batch][acc_stride]; the
 * softmax weight of every live token, summed over the query heads, is added
 * to it (acc_stride >= every seq_len).
 * Returns 0 or -1 on bad arguments. */
int orc_decode(const orc_cache* segs, const orc_view* views, int32_t nseg,
               const float* q, int32_t batch, int32_t num_q_heads,
               float sm_scale, float tau_low, int32_t split_tokens,
               double* out, uint8_t* skip, double* score_acc, int32_t acc_stride);

/* orc_decode with the near-threshold skip decisions resolved: a pair whose
 * exact margin |exp(s - m) - tau_low * L| is at most band * tau_low * L can
 * go either way in finite precision; for it the decision in given (layout of
 * skip; NULL keeps the exact one) is taken and ambiguous (same layout, may
 * be NULL, filled with 1 where a pair is ambiguous and left alone elsewhere)
 * records it.  margin (may be NULL, layout of skip, fp64) receives each live
 * pair's relative margin (exp(s - m) - tau_low * L) / (tau_low * L) when
 * tau_low > 0.  band >= 0. */
int orc_decode_resolved(const orc_cache* segs, const orc_view* views, int32_t nseg,
                        const float* q, int32_t batch, int32_t num_q_heads,
                        float sm_scale, float tau_low, int32_t split_tokens,
                        double* out, uint8_t* skip, const uint8_t* given, double band, uint8_t* ambiguous,
                        double* margin, double* score_acc, int32_t acc_stride);

/* Tier update.  src: K6V6 cache + view.  scores fp32 [batch][scores_stride].
 * Writes tiers uint8 [batch][scores_stride] (0 low, 1 mid, 2 high; entries
 * past the sequence length are left untouched), compacts HIGH tokens into
 * dst_h (K6V6) and MID tokens into dst_m (K6V4), both addressed through
 * their own block tables from position 0, and returns the counts. */
int orc_tier_update(const orc_cache* src, const orc_view* src_view,
                    const float* scores, int32_t scores_stride,
                    float tau_low, float tau_high,
                    const orc_cache* dst_h, const int32_t* h_block_table, int32_t h_max_blocks,
                    const orc_cache* dst_m, const int32_t* m_block_table, int32_t m_max_blocks,
                    int32_t* n_high, int32_t* n_mid, uint8_t* tiers, int32_t batch);

/* Re-tiering of a tiered cache {h: K6V6, m: K6V4} with fresh scores
 * ([batch][h_stride], [batch][m_stride]) into new segments dst_h (K6V6) and
 * dst_m (K6V4): HIGH tokens of h with score >= tau_high stay HIGH; tokens of
 * h with tau_low <= score < tau_high are demoted to MID (V requantised);
 * tokens of m with score >= tau_low stay MID (never promoted); tokens with
 * score < tau_low are evicted.  dst_m holds the kept MID tokens first, then
 * the demoted ones, each in token order.  h_tiers, m_tiers receive the new
 * tier of every source token; n_high, n_mid the new counts.  Returns 0, or
 * -1 on bad arguments (including a destination without room). */
int orc_retier(const orc_cache* h, const orc_view* h_view, const float* h_scores, int32_t h_stride,
               const orc_cache* m, const orc_view* m_view, const float* m_scores, int32_t m_stride,
               float tau_low, float tau_high,
               const orc_cache* dst_h, const int32_t* dh_bt, int32_t dh_max_blocks,
               const orc_cache* dst_m, const int32_t* dm_bt, int32_t dm_max_blocks,
               int32_t* n_high, int32_t* n_mid, uint8_t* h_tiers, uint8_t* m_tiers, int32_t batch);

/* Thresholds from the 4-bit and 6-bit quantisation error bounds for n live
 * tokens: tau_low = eps4/n, tau_high = (eps4/eps6)/n, eps_b = 1/(2(2^b-1)). */
void orc_default_thresholds(int32_t n_tokens, float* tau_low, float* tau_high);

/* Threads an OpenMP parallel region of the oracle runs with (1 when built
 * without OpenMP): the core count a timing of the oracle states. */
int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
