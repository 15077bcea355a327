// lkv_internal.h -- shared declarations of the HIP library (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lkv.h"

namespace lkv {

constexpr int BT = LKV_BLOCK_TOKENS;  // tokens per block / chunk

// Resolved cache format: byte offsets of the six chunk sections.
struct Fmt {
    int32_t D, g, kb, vb, H, ngroups;
    int32_t fp16;                                     // k_bits == v_bits == 16
    int32_t off_kc, off_vc, off_ks, off_vs, off_kz, off_vz;
    int32_t krow;                                     // bytes of one K token row
    int32_t vrow;                                     // bytes of one V channel row
    int64_t chunk;                                    // bytes of one chunk
    int32_t k_norm;                                   // direction-preserving K: factors at off_kn
    int32_t off_kn;                                   // fp32 [64] norm factors, after the six sections
};

// Fills f from a cache descriptor; returns LKV_OK, LKV_EINVAL or
// LKV_EUNSUPPORTED.
int make_fmt(const lkv_cache* c, Fmt* f);

// One segment of a decode call, as the split kernel sees it.
struct SegArgs {
    Fmt f;
    const uint8_t* pool;
    const int32_t* block_table;
    const int32_t* seq_lens;
    int32_t max_blocks;
    int32_t len_cap;       // the view's max_len (<= max_blocks * 64): lengths are clamped to it, so
                           // an out-of-contract length never reaches past the grid or the score rows
    int32_t n_splits;      // splits of this segment in the grid
    int32_t split_base;    // index of its first split in the partials
    // optional: every live token's base-2 score per query head, into rows
    // scores[b * num_q_heads + h][score_stride] from column tok_base
    // (multiples of 64); null when the call wants no scores
    float* scores;
    int32_t score_stride;
    int32_t tok_base;
    // query tokens per sequence: grid entry e is query token e % q_per_seq of
    // sequence e / q_per_seq; when causal (the segment holding the new
    // tokens) that entry reads all but the q_per_seq - 1 - e % q_per_seq
    // newest tokens
    int32_t q_per_seq;
    int32_t causal;
    // optional (test entry point only): one bit per (grid entry, query
    // head, score column), set when the token's V term is skipped; rows of
    // mask_stride words, cleared by the caller; null otherwise
    uint32_t* skip_mask;
    int32_t mask_stride;
};

// Records a skipped (token, head) pair in a skip-mask row (bit col).
__device__ __forceinline__ void mark_skipped(uint32_t* row, int col)
{
    atomicOr(row + (col >> 5), 1u << (col & 31));
}

// Block-table row and length that grid entry e reads in segment s (the
// length before clamping to the table).
__device__ __forceinline__ int entry_seq(const SegArgs& s, int e) { return e / s.q_per_seq; }
__device__ __forceinline__ int entry_len(const SegArgs& s, int e)
{
    const int len = s.seq_lens[e / s.q_per_seq];
    return s.causal ? len - (s.q_per_seq - 1 - e % s.q_per_seq) : len;
}

// cu_new null: one row per sequence (row b) at position min(start_pos[b],
// len_cap) - 1, start_pos holding lengths that count the row.
hipError_t launch_append(const Fmt& f, uint8_t* pool, const void* k, const void* v, int dtype,
                         const int32_t* cu_new, const int32_t* start_pos, const int32_t* block_table,
                         int32_t max_blocks, int32_t batch, int32_t max_new, hipStream_t stream,
                         int32_t len_cap = 0);

// The matrix-core split kernel that also appends each sequence's newest row
// (lkv_append_decode); false when the format, shape or input alignment has
// no such kernel.
bool launch_append_decode_mfma(const SegArgs& s, const void* q, int q_dtype, int32_t batch, int32_t num_q_heads,
                               float sm_scale, float tau_low, int32_t split_tokens, int32_t total_splits,
                               float* partials, const void* k_new, const void* v_new, int kv_dtype,
                               hipStream_t stream, hipError_t* err, float* out = nullptr,
                               uint32_t* counters = nullptr, bool ragged = false);

// The one-launch decode step of a tiered cache: HIGH (K6V6) takes the new
// rows, both segments are read and the splits merged in the kernel; false
// when the pair or the shape has no such kernel.
bool launch_append_decode_tiered_merged(const SegArgs& high, const SegArgs& mid, const void* q, int q_dtype,
                                        int32_t batch, int32_t num_q_heads, float sm_scale, float tau_low,
                                        int32_t split_tokens, int32_t total_splits, float* partials,
                                        const void* k_new, const void* v_new, int kv_dtype, hipStream_t stream,
                                        hipError_t* err, float* out, uint32_t* counters);

// Partials: fp32 [batch][Hq][total_splits][D + 2] = (o[D], m, L).
hipError_t launch_decode_split(const SegArgs& s, const void* q, int q_dtype, int32_t batch,
                               int32_t num_q_heads, float sm_scale, float tau_low,
                               int32_t split_tokens, int32_t total_splits, float* partials,
                               hipStream_t stream);

// Matrix-core split kernel: launches and returns true when the format and
// shape have one (bf16 Q, D 128, g 64, K6, V4 or V6, G 4 or 8).
bool launch_decode_split_mfma(const SegArgs& s, const void* q, int q_dtype, int32_t batch, int32_t num_q_heads,
                              float sm_scale, float tau_low, int32_t split_tokens, int32_t total_splits,
                              float* partials, hipStream_t stream, hipError_t* err);

// Both segments of a tiered cache ({HIGH K6V6, MID K6V4}) in one matrix-core
// launch; false when either segment has no matrix-core kernel.
bool launch_decode_split_mfma_tiered(const SegArgs& high, const SegArgs& mid, const void* q, int q_dtype,
                                     int32_t batch, int32_t num_q_heads, float sm_scale, float tau_low,
                                     int32_t split_tokens, int32_t total_splits, float* partials,
                                     hipStream_t stream, hipError_t* err);

// Matrix-core split kernel of the fp16 format: launches and returns true for
// D 128, bf16 or fp32 Q, G 4 or 8.
bool launch_decode_split_f16(const SegArgs& s, const void* q, int q_dtype, int32_t batch, int32_t num_q_heads,
                             float sm_scale, float tau_low, int32_t split_tokens, int32_t total_splits,
                             float* partials, hipStream_t stream, hipError_t* err);

// What the merge reads and writes: partials [B][Hq][total_splits][D + 2]
// (splits without tokens hold only m = -inf, L = 0), out [B][Hq][D].
struct CombineArgs {
    const float* part;
    float* out;
    int32_t num_q_heads;
    int32_t total_splits;
    float* ml;             // optional: (M, 1 / L) of every (sequence, head), base 2
    // optional (one segment, a row per sequence): the sequences' lengths, so
    // that splits past a sequence's end, whose (m, L) = (-inf, 0), are not
    // read at all; null: every split is read
    const int32_t* lens;
    int32_t len_cap;
    int32_t split_tokens;
};

// Accumulated attention scores: for every live token j of segment s of
// sequence b, acc[s][b][j] += sum_h 2^(score[b][h][tok_base_s + j] - M_bh) / L_bh.
struct ScoreAccArgs {
    const float* scores;
    int32_t score_stride;
    const float* ml;
    int32_t num_q_heads;
    int32_t batch;
    int32_t nseg;
    const int32_t* lens[2];
    int32_t len_cap[2];
    int32_t tok_base[2];
    float* acc;
    int32_t acc_stride;
};

hipError_t launch_score_accumulate(const ScoreAccArgs& a, hipStream_t stream);

hipError_t launch_decode_combine(const CombineArgs& a, int32_t batch, int32_t D, hipStream_t stream);

// p[0 .. n) = v on the stream (a kernel, not a memset node).
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t stream);

// Streaming read of `bytes` (a multiple of 16, 16-byte aligned) of a device
// buffer; writes sink[0] only if the buffer's words fold to a fixed value.
hipError_t launch_hbm_read_probe(const void* buf, int64_t bytes, bool nontemporal, uint32_t* sink, hipStream_t stream);

// A source segment of a tier scan and a destination segment.
struct TierSource {
    Fmt f;
    const uint8_t* pool;
    const int32_t* block_table;
    const int32_t* view_lens;
    int32_t max_blocks;
    int32_t max_len;
    const float* scores;   // [batch][stride]
    int32_t stride;
    uint8_t* tiers;        // [batch][stride]
    int32_t max_tier;      // 2, or 1 for a MID source (never promoted)
};
struct TierDest {
    Fmt f;
    uint8_t* pool;
    const int32_t* block_table;
    int32_t max_blocks;
};

// Tier update (one K6V6 source) or re-tiering (sources {MID, HIGH}, in that
// order).  workspace: tiering_workspace_bytes(), 8-byte aligned.
hipError_t launch_tiering(const TierSource* src, int nsrc, float tau_low, float tau_high, const TierDest& h,
                          const TierDest& m, int32_t* n_high, int32_t* n_mid, int32_t batch, void* workspace,
                          hipStream_t stream);

// Scan chunks of a scores row of `stride` tokens (2048 tokens each, at least one).
inline int32_t tier_chunks(int32_t stride) { return stride > 0 ? (stride + 2047) / 2048 : 1; }

// 64-token blocks of a scores row (at least one).
inline int32_t tier_blocks(int32_t stride) { return stride > 0 ? (stride + BT - 1) / BT : 1; }

// The (HIGH, MID) int32 counts of every scan chunk of every source, then
// the (HIGH, MID) destination positions of every 64-token block of every
// source, then (in-place compaction) a ticket counter padded to 8 bytes and
// a uint32 read count per 64-token block of the longest source.
inline int64_t tiering_workspace_bytes(int32_t batch, const int32_t* strides, int nsrc)
{
    int64_t chunks = 0, blocks = 0, widest = 0;
    for (int i = 0; i < nsrc; i++) {
        chunks += tier_chunks(strides[i]);
        blocks += tier_blocks(strides[i]);
        widest = tier_blocks(strides[i]) > widest ? tier_blocks(strides[i]) : widest;
    }
    return (int64_t)batch * (chunks + blocks) * 8 + 8 + (int64_t)batch * widest * 4;
}

}  // namespace lkv
