// api.cpp -- the C ABI of include/lkv.h: host-side validation, split plans
// and kernel launches.  No allocation, no synchronisation, no global state.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "lkv_internal.h"

namespace lkv {

static int64_t pad128(int64_t x) { return (x + 127) / 128 * 128; }

int make_fmt(const lkv_cache* c, Fmt* f)
{
    if (!c) return LKV_EINVAL;
    int64_t off[7];
    const int st = lkv_chunk_layout(c->head_dim, c->group_size, c->k_bits, c->v_bits, off);
    if (st != LKV_OK) return st;
    if (c->block_tokens != BT) return LKV_EUNSUPPORTED;
    if (c->num_kv_heads < 1 || c->num_blocks < 1 || !c->pool) return LKV_EINVAL;
    if ((uintptr_t)c->pool % 256 != 0) return LKV_EINVAL;
    f->D = c->head_dim;
    f->g = c->group_size;
    f->kb = c->k_bits;
    f->vb = c->v_bits;
    f->H = c->num_kv_heads;
    f->fp16 = c->k_bits == 16;
    f->ngroups = f->fp16 ? 0 : c->head_dim / c->group_size;
    f->off_kc = (int32_t)off[0];
    f->off_vc = (int32_t)off[1];
    f->off_ks = (int32_t)off[2];
    f->off_vs = (int32_t)off[3];
    f->off_kz = (int32_t)off[4];
    f->off_vz = (int32_t)off[5];
    f->chunk = off[6];
    f->krow = c->head_dim * c->k_bits / 8;
    f->vrow = BT * c->v_bits / 8;
    f->k_norm = c->k_norm != 0;
    f->off_kn = (int32_t)off[6];
    if (f->k_norm) {
        if (f->fp16) return LKV_EUNSUPPORTED;
        f->chunk += BT * 4;  // one fp32 factor per slot
    }
    return LKV_OK;
}

static bool g_supported(int G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }

// Checks shared by the decode entry points; fills one Fmt per segment.
static int check_decode(const lkv_cache* segs, const lkv_view* views, int32_t nseg, int32_t batch,
                        int32_t num_q_heads, Fmt* f)
{
    if (!segs || !views || nseg < 1 || nseg > 2 || batch < 0 || num_q_heads < 1) return LKV_EINVAL;
    for (int s = 0; s < nseg; s++) {
        const int st = make_fmt(&segs[s], &f[s]);
        if (st != LKV_OK) return st;
        if (f[s].D != f[0].D || f[s].H != f[0].H) return LKV_EINVAL;
        const lkv_view& v = views[s];
        if (v.max_blocks < 1 || v.max_len < 0 || (int64_t)v.max_len > (int64_t)v.max_blocks * BT)
            return LKV_EINVAL;
        if (batch > 0 && (!v.block_table || !v.seq_lens)) return LKV_EINVAL;
    }
    if (num_q_heads % f[0].H != 0) return LKV_EINVAL;
    if (!g_supported(num_q_heads / f[0].H)) return LKV_EUNSUPPORTED;
    return LKV_OK;
}

static int32_t splits_of(int32_t max_len, int32_t split_tokens)
{
    return (max_len + split_tokens - 1) / split_tokens;
}

static int64_t total_splits(const lkv_view* views, int32_t nseg, int32_t split_tokens)
{
    int64_t n = 0;
    for (int s = 0; s < nseg; s++) n += splits_of(views[s].max_len, split_tokens);
    return n;
}

static int64_t align256(int64_t n) { return (n + 255) / 256 * 256; }

// Columns of the score rows: every segment's max_len rounded up to 64.
static int32_t score_cols(const lkv_view* views, int32_t nseg)
{
    int32_t n = 0;
    for (int s = 0; s < nseg; s++) n += (views[s].max_len + BT - 1) / BT * BT;
    return n;
}

// Host checks of the split stage (every one of them runs before a launch);
// fills one Fmt per segment.  batch counts grid entries.
static int check_split(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* q, int32_t q_dtype,
                       int32_t batch, int32_t num_q_heads, float sm_scale, float tau_low, int32_t split_tokens,
                       const void* workspace, size_t workspace_bytes, Fmt* f)
{
    const int st = check_decode(segs, views, nseg, batch, num_q_heads, f);
    if (st != LKV_OK) return st;
    if (q_dtype != LKV_F32 && q_dtype != LKV_BF16) return LKV_EINVAL;
    if (split_tokens <= 0 || split_tokens % BT != 0) return LKV_EINVAL;
    if (!std::isfinite(sm_scale) || std::isnan(tau_low)) return LKV_EINVAL;
    const int64_t need = (int64_t)batch * num_q_heads * total_splits(views, nseg, split_tokens) * (f[0].D + 2) * 4;
    if ((int64_t)workspace_bytes < need) return LKV_EINVAL;
    if (batch == 0) return LKV_OK;
    if (!q || (need > 0 && !workspace) || (uintptr_t)workspace % 16 != 0) return LKV_EINVAL;
    return LKV_OK;
}

// The kernels' view of the segments; returns the total split count.
static int32_t seg_args(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const Fmt* f,
                        int32_t split_tokens, float* scores, int32_t score_stride, int32_t q_per_seq,
                        uint32_t* skip_mask, int32_t mask_stride, SegArgs* a);

// Split stage; scores (optional) receives the base-2 score rows.  batch
// counts grid entries: sequences times q_per_seq query tokens.
static int split_impl(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* q, int32_t q_dtype,
                      int32_t batch, int32_t num_q_heads, float sm_scale, float tau_low, int32_t split_tokens,
                      void* workspace, size_t workspace_bytes, void* stream, float* scores, int32_t score_stride,
                      int32_t q_per_seq = 1, uint32_t* skip_mask = nullptr, int32_t mask_stride = 0);

// Merge stage; ml (optional) receives (M, 1 / L) per (sequence, head).
// per_seq: the rows are the views' sequences (not multi-token entries), so a
// one-segment merge of a ragged batch can skip the splits past each
// sequence's end.
static int combine_impl(const lkv_cache* segs, const lkv_view* views, int32_t nseg, int32_t batch,
                        int32_t num_q_heads, int32_t split_tokens, float* out, const void* workspace,
                        size_t workspace_bytes, void* stream, float* ml, bool per_seq = true);

// The view's host hint says the batch is ragged: its total length is known
// and below batch x max_len.
static bool ragged_hint(const lkv_view* view, int32_t batch)
{
    return view->sum_len > 0 && view->sum_len < (int64_t)batch * view->max_len;
}

}  // namespace lkv

using namespace lkv;

extern "C" {

const char* lkv_status_string(int status)
{
    switch (status) {
    case LKV_OK: return "ok";
    case LKV_EINVAL: return "invalid argument";
    case LKV_EUNSUPPORTED: return "unsupported format or shape";
    case LKV_EHIP: return "HIP launch failed";
    case LKV_ESCRATCH: return "the call needs more than the library's static decode scratch";
    default: return "unknown status";
    }
}

int lkv_chunk_layout(int32_t head_dim, int32_t group_size, int32_t k_bits, int32_t v_bits, int64_t off[7])
{
    if (!off) return LKV_EINVAL;
    if (head_dim != 64 && head_dim != 128) return LKV_EUNSUPPORTED;
    const bool fp16 = k_bits == 16 && v_bits == 16;
    const bool q_ok = (k_bits == 4 || k_bits == 6) && (v_bits == 4 || v_bits == 6);
    if (!fp16 && !q_ok) return LKV_EUNSUPPORTED;
    if (!fp16 && !(group_size == 16 || group_size == 32 || group_size == 64)) return LKV_EUNSUPPORTED;
    if (!fp16 && head_dim % group_size != 0) return LKV_EUNSUPPORTED;
    const int64_t ng = fp16 ? 0 : head_dim / group_size;
    const int64_t sz[6] = {(int64_t)BT * head_dim * k_bits / 8, (int64_t)head_dim * BT * v_bits / 8,
                           ng * BT * 4, ng * BT * 4, ng * BT, ng * BT};
    int64_t at = 0;
    for (int i = 0; i < 6; i++) {
        off[i] = at;
        at += pad128(sz[i]);
    }
    off[6] = at;
    return LKV_OK;
}

int lkv_quant_append(const lkv_cache* cache, const void* k, const void* v, int32_t dtype,
                     const int32_t* cu_new, const int32_t* start_pos, const int32_t* block_table,
                     int32_t max_blocks, int32_t batch, int32_t max_new, void* stream)
{
    Fmt f;
    const int st = make_fmt(cache, &f);
    if (st != LKV_OK) return st;
    if (batch < 0 || max_new < 0 || max_blocks < 1) return LKV_EINVAL;
    if (dtype != LKV_F32 && dtype != LKV_BF16 && dtype != LKV_F16) return LKV_EINVAL;
    if (batch == 0 || max_new == 0) return LKV_OK;
    if (!k || !v || !cu_new || !start_pos || !block_table) return LKV_EINVAL;
    if (f.k_norm) {  // the norm factors come from the quantised kernel, which needs P-element alignment
        const uintptr_t need = (uintptr_t)(f.D / 64) * (dtype == LKV_F32 ? 4 : 2);
        if ((uintptr_t)k % need != 0 || (uintptr_t)v % need != 0) return LKV_EUNSUPPORTED;
    }
    const hipError_t e = launch_append(f, (uint8_t*)cache->pool, k, v, dtype, cu_new, start_pos, block_table,
                                       max_blocks, batch, max_new, (hipStream_t)stream);
    return e == hipSuccess ? LKV_OK : LKV_EHIP;
}

int lkv_decode_plan(const lkv_cache* segs, const lkv_view* views, int32_t nseg, int32_t batch,
                    int32_t num_q_heads, int32_t* split_tokens)
{
    Fmt f[2];
    if (!split_tokens) return LKV_EINVAL;
    const int st = check_decode(segs, views, nseg, batch, num_q_heads, f);
    if (st != LKV_OK) return st;
    // Aim at about 2048 single-wave work items (8 per compute unit on a
    // 256-CU part, two resident waves per SIMD), never fewer than one
    // 64-token block nor more than 64 blocks per split.
    constexpr int64_t ITEMS = 2048;
    bool hinted = false;
    for (int s = 0; s < nseg; s++) hinted |= views[s].sum_len > 0;
    int64_t per = 1;
    if (!hinted) {
        // every sequence counted at max_len: equal splits fill the items
        int64_t blocks = 0;
        for (int s = 0; s < nseg; s++) blocks += (int64_t)batch * f[0].H * ((views[s].max_len + BT - 1) / BT);
        per = (blocks + ITEMS - 1) / ITEMS;
    } else {
        // a ragged batch: each sequence's last split is partial, so a split
        // size p gives at most H * (total blocks / p + batch) splits with
        // work; take the smallest p whose count fits in one round of items
        for (per = 1; per < 64; per++) {
            int64_t items = 0;
            for (int s = 0; s < nseg; s++) {
                const int64_t dense = (int64_t)batch * ((views[s].max_len + BT - 1) / BT);
                const int64_t blocks =
                    views[s].sum_len > 0 ? std::min(dense, (views[s].sum_len + BT - 1) / BT) : dense;
                items += (int64_t)f[0].H * ((blocks + per - 1) / per + batch);
            }
            if (items <= ITEMS) break;
        }
    }
    if (per < 1) per = 1;
    if (per > 64) per = 64;
    *split_tokens = (int32_t)(per * BT);
    return LKV_OK;
}

int lkv_decode_plan_lens(const lkv_cache* cache, const lkv_view* view, const int32_t* host_lens, int32_t batch,
                         int32_t num_q_heads, int32_t* split_tokens)
{
    const int st = lkv_decode_plan(cache, view, 1, batch, num_q_heads, split_tokens);
    if (st != LKV_OK) return st;
    if (batch > 0 && !host_lens) return LKV_EINVAL;
    // the decode step's compact order runs only the splits with tokens (an
    // empty sequence counts one): a ragged batch of at most 64 sequences in
    // a format with the fused matrix-core step
    const int G = num_q_heads / cache->num_kv_heads;
    const bool compact = batch <= 64 && ragged_hint(view, batch) && cache->head_dim == 128 && cache->k_bits == 6 &&
                         (cache->v_bits == 4 || cache->v_bits == 6) && !cache->k_norm && (G == 4 || G == 8);
    if (!compact) return LKV_OK;
    // the smallest split whose items fit in one round of 2048, counted exactly
    constexpr int64_t ITEMS = 2048;
    int64_t per = 1;
    for (; per < 64; per++) {
        int64_t items = 0;
        for (int b = 0; b < batch; b++) {
            const int64_t len = std::max<int64_t>(0, std::min<int64_t>(host_lens[b], view->max_len));
            items += cache->num_kv_heads * std::max<int64_t>(1, (len + per * BT - 1) / (per * BT));
        }
        if (items <= ITEMS) break;
    }
    *split_tokens = (int32_t)(per * BT);
    return LKV_OK;
}

int64_t lkv_decode_workspace_bytes(const lkv_cache* segs, const lkv_view* views, int32_t nseg, int32_t batch,
                                   int32_t num_q_heads, int32_t split_tokens)
{
    Fmt f[2];
    const int st = check_decode(segs, views, nseg, batch, num_q_heads, f);
    if (st != LKV_OK) return st;
    if (split_tokens <= 0 || split_tokens % BT != 0) return LKV_EINVAL;
    return (int64_t)batch * num_q_heads * total_splits(views, nseg, split_tokens) * (f[0].D + 2) * 4;
}

}  // extern "C"

namespace lkv {

static int split_impl(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* q, int32_t q_dtype,
                      int32_t batch, int32_t num_q_heads, float sm_scale, float tau_low, int32_t split_tokens,
                      void* workspace, size_t workspace_bytes, void* stream, float* scores, int32_t score_stride,
                      int32_t q_per_seq, uint32_t* skip_mask, int32_t mask_stride)
{
    Fmt f[2];
    const int st = check_split(segs, views, nseg, q, q_dtype, batch, num_q_heads, sm_scale, tau_low, split_tokens,
                               workspace, workspace_bytes, f);
    if (st != LKV_OK || batch == 0) return st;
    SegArgs a[2];
    const int32_t tot = seg_args(segs, views, nseg, f, split_tokens, scores, score_stride, q_per_seq, skip_mask,
                                 mask_stride, a);
    hipError_t e;
    if (nseg == 2 && launch_decode_split_mfma_tiered(a[0], a[1], q, q_dtype, batch, num_q_heads, sm_scale, tau_low,
                                                     split_tokens, tot, (float*)workspace, (hipStream_t)stream, &e))
        return e == hipSuccess ? LKV_OK : LKV_EHIP;
    for (int s = 0; s < nseg; s++) {
        e = launch_decode_split(a[s], q, q_dtype, batch, num_q_heads, sm_scale, tau_low, split_tokens, tot,
                                (float*)workspace, (hipStream_t)stream);
        if (e != hipSuccess) return LKV_EHIP;
    }
    return LKV_OK;
}

static int32_t seg_args(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const Fmt* f,
                        int32_t split_tokens, float* scores, int32_t score_stride, int32_t q_per_seq,
                        uint32_t* skip_mask, int32_t mask_stride, SegArgs* a)
{
    int32_t base = 0;
    for (int s = 0; s < nseg; s++) {
        a[s].f = f[s];
        a[s].pool = (const uint8_t*)segs[s].pool;
        a[s].block_table = views[s].block_table;
        a[s].seq_lens = views[s].seq_lens;
        a[s].max_blocks = views[s].max_blocks;
        a[s].len_cap = views[s].max_len;
        a[s].n_splits = splits_of(views[s].max_len, split_tokens);
        a[s].split_base = base;
        base += a[s].n_splits;
        a[s].scores = scores;
        a[s].score_stride = score_stride;
        a[s].tok_base = s == 0 ? 0 : (views[0].max_len + BT - 1) / BT * BT;
        a[s].q_per_seq = q_per_seq;
        a[s].causal = q_per_seq > 1 && s == 0;  // the new tokens are the first segment's tail
        a[s].skip_mask = skip_mask;
        a[s].mask_stride = mask_stride;
    }
    return base;
}

static int combine_impl(const lkv_cache* segs, const lkv_view* views, int32_t nseg, int32_t batch,
                        int32_t num_q_heads, int32_t split_tokens, float* out, const void* workspace,
                        size_t workspace_bytes, void* stream, float* ml, bool per_seq)
{
    Fmt f[2];
    const int st = check_decode(segs, views, nseg, batch, num_q_heads, f);
    if (st != LKV_OK) return st;
    if (split_tokens <= 0 || split_tokens % BT != 0) return LKV_EINVAL;
    const int64_t tot = total_splits(views, nseg, split_tokens);
    const int64_t need = (int64_t)batch * num_q_heads * tot * (f[0].D + 2) * 4;
    if ((int64_t)workspace_bytes < need) return LKV_EINVAL;
    if (batch == 0) return LKV_OK;
    if (!out || (need > 0 && !workspace)) return LKV_EINVAL;
    CombineArgs ca;
    ca.part = (const float*)workspace;
    ca.out = out;
    ca.num_q_heads = num_q_heads;
    ca.total_splits = (int32_t)tot;
    ca.ml = ml;
    // a ragged batch (the host's total length below batch x max_len): its
    // merge reads only the splits that hold tokens (one length load per row
    // first, which a uniform batch would pay for nothing)
    const bool skip = per_seq && nseg == 1 && ragged_hint(&views[0], batch);
    ca.lens = skip ? views[0].seq_lens : nullptr;
    ca.len_cap = skip ? views[0].max_len : 0;
    ca.split_tokens = split_tokens;
    const hipError_t e = launch_decode_combine(ca, batch, f[0].D, (hipStream_t)stream);
    return e == hipSuccess ? LKV_OK : LKV_EHIP;
}

}  // namespace lkv

extern "C" {

int lkv_decode_split(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* q, int32_t q_dtype,
                     int32_t batch, int32_t num_q_heads, float sm_scale, float tau_low, int32_t split_tokens,
                     void* workspace, size_t workspace_bytes, void* stream)
{
    return split_impl(segs, views, nseg, q, q_dtype, batch, num_q_heads, sm_scale, tau_low, split_tokens, workspace,
                      workspace_bytes, stream, nullptr, 0);
}

int lkv_decode_combine(const lkv_cache* segs, const lkv_view* views, int32_t nseg, int32_t batch,
                       int32_t num_q_heads, int32_t split_tokens, float* out, const void* workspace,
                       size_t workspace_bytes, void* stream)
{
    return combine_impl(segs, views, nseg, batch, num_q_heads, split_tokens, out, workspace, workspace_bytes, stream,
                        nullptr);
}

int64_t lkv_decode_scores_workspace_bytes(const lkv_cache* segs, const lkv_view* views, int32_t nseg,
                                          int32_t batch, int32_t num_q_heads, int32_t split_tokens)
{
    const int64_t part = lkv_decode_workspace_bytes(segs, views, nseg, batch, num_q_heads, split_tokens);
    if (part < 0) return part;
    return align256(part) + align256((int64_t)batch * num_q_heads * score_cols(views, nseg) * 4) +
           (int64_t)batch * num_q_heads * 8;
}

int lkv_decode_attn_scores(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* q,
                           int32_t q_dtype, int32_t batch, int32_t num_q_heads, float sm_scale, float tau_low,
                           int32_t split_tokens, float* out, float* score_acc, int32_t acc_stride, void* workspace,
                           size_t workspace_bytes, void* stream)
{
    if (split_tokens == 0) {
        const int st = lkv_decode_plan(segs, views, nseg, batch, num_q_heads, &split_tokens);
        if (st != LKV_OK) return st;
    }
    const int64_t need = lkv_decode_scores_workspace_bytes(segs, views, nseg, batch, num_q_heads, split_tokens);
    if (need < 0) return (int)need;
    if ((int64_t)workspace_bytes < need) return LKV_EINVAL;
    for (int s = 0; s < nseg; s++)
        if (acc_stride < views[s].max_len) return LKV_EINVAL;
    if (batch == 0) return LKV_OK;
    if (!out || !score_acc || !workspace || (uintptr_t)workspace % 256 != 0) return LKV_EINVAL;
    const int64_t part = align256(lkv_decode_workspace_bytes(segs, views, nseg, batch, num_q_heads, split_tokens));
    const int32_t cols = score_cols(views, nseg);
    float* scores = (float*)((uint8_t*)workspace + part);
    float* ml = (float*)((uint8_t*)workspace + part + align256((int64_t)batch * num_q_heads * cols * 4));
    int st = split_impl(segs, views, nseg, q, q_dtype, batch, num_q_heads, sm_scale, tau_low, split_tokens,
                        workspace, (size_t)part, stream, scores, cols);
    if (st != LKV_OK) return st;
    st = combine_impl(segs, views, nseg, batch, num_q_heads, split_tokens, out, workspace, (size_t)part, stream, ml);
    if (st != LKV_OK) return st;
    ScoreAccArgs sa;
    sa.scores = scores;
    sa.score_stride = cols;
    sa.ml = ml;
    sa.num_q_heads = num_q_heads;
    sa.batch = batch;
    sa.nseg = nseg;
    for (int s = 0; s < 2; s++) {
        const bool on = s < nseg;
        sa.lens[s] = on ? views[s].seq_lens : nullptr;
        sa.len_cap[s] = on ? views[s].max_len : 0;
        sa.tok_base[s] = s == 0 ? 0 : (views[0].max_len + BT - 1) / BT * BT;
    }
    sa.acc = score_acc;
    sa.acc_stride = acc_stride;
    return launch_score_accumulate(sa, (hipStream_t)stream) == hipSuccess ? LKV_OK : LKV_EHIP;
}

int lkv_decode_attn(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* q, int32_t q_dtype,
                    int32_t batch, int32_t num_q_heads, float sm_scale, float tau_low, int32_t split_tokens,
                    float* out, void* workspace, size_t workspace_bytes, void* stream)
{
    if (split_tokens == 0) {
        const int st = lkv_decode_plan(segs, views, nseg, batch, num_q_heads, &split_tokens);
        if (st != LKV_OK) return st;
    }
    if (batch > 0 && !out) return LKV_EINVAL;
    int st = lkv_decode_split(segs, views, nseg, q, q_dtype, batch, num_q_heads, sm_scale, tau_low, split_tokens,
                              workspace, workspace_bytes, stream);
    if (st != LKV_OK) return st;
    return lkv_decode_combine(segs, views, nseg, batch, num_q_heads, split_tokens, out, workspace, workspace_bytes,
                              stream);
}

int lkv_append_split(const lkv_cache* cache, const lkv_view* view, const void* k_new, const void* v_new,
                     int32_t kv_dtype, const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                     float sm_scale, float tau_low, int32_t split_tokens, void* workspace, size_t workspace_bytes,
                     void* stream)
{
    Fmt f[2];
    int st = check_split(cache, view, 1, q, q_dtype, batch, num_q_heads, sm_scale, tau_low, split_tokens, workspace,
                         workspace_bytes, f);
    if (st != LKV_OK) return st;
    if (kv_dtype != LKV_F32 && kv_dtype != LKV_BF16 && kv_dtype != LKV_F16) return LKV_EINVAL;
    if (batch == 0) return LKV_OK;
    if (!k_new || !v_new) return LKV_EINVAL;
    if (f[0].k_norm) {  // as lkv_quant_append: the norm factors need P-element alignment
        const uintptr_t need = (uintptr_t)(f[0].D / 64) * (kv_dtype == LKV_F32 ? 4 : 2);
        if ((uintptr_t)k_new % need != 0 || (uintptr_t)v_new % need != 0) return LKV_EUNSUPPORTED;
    }
    SegArgs a[2];
    const int32_t tot = seg_args(cache, view, 1, f, split_tokens, nullptr, 0, 1, nullptr, 0, a);
    hipError_t e;
    if (!launch_append_decode_mfma(a[0], q, q_dtype, batch, num_q_heads, sm_scale, tau_low, split_tokens, tot,
                                   (float*)workspace, k_new, v_new, kv_dtype, (hipStream_t)stream, &e, nullptr,
                                   nullptr, ragged_hint(view, batch))) {
        // no fused kernel for this format: the append kernel (one row per
        // sequence at its last position), then the split kernel
        e = launch_append(f[0], (uint8_t*)cache->pool, k_new, v_new, kv_dtype, nullptr, view->seq_lens,
                          view->block_table, view->max_blocks, batch, 1, (hipStream_t)stream, view->max_len);
        if (e != hipSuccess) return LKV_EHIP;
        e = launch_decode_split(a[0], q, q_dtype, batch, num_q_heads, sm_scale, tau_low, split_tokens, tot,
                                (float*)workspace, (hipStream_t)stream);
    }
    return e == hipSuccess ? LKV_OK : LKV_EHIP;
}

int lkv_append_decode(const lkv_cache* cache, const lkv_view* view, const void* k_new, const void* v_new,
                      int32_t kv_dtype, const void* q, int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                      float sm_scale, float tau_low, int32_t split_tokens, float* out, void* workspace,
                      size_t workspace_bytes, void* stream)
{
    if (split_tokens == 0) {
        const int st = lkv_decode_plan(cache, view, 1, batch, num_q_heads, &split_tokens);
        if (st != LKV_OK) return st;
    }
    if (batch > 0 && !out) return LKV_EINVAL;
    const int st = lkv_append_split(cache, view, k_new, v_new, kv_dtype, q, q_dtype, batch, num_q_heads, sm_scale,
                                    tau_low, split_tokens, workspace, workspace_bytes, stream);
    if (st != LKV_OK) return st;
    return lkv_decode_combine(cache, view, 1, batch, num_q_heads, split_tokens, out, workspace, workspace_bytes,
                              stream);
}

int lkv_append_decode_merged(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* k_new,
                             const void* v_new, int32_t kv_dtype, const void* q, int32_t q_dtype, int32_t batch,
                             int32_t num_q_heads, float sm_scale, float tau_low, int32_t split_tokens, float* out,
                             uint32_t* counters, void* workspace, size_t workspace_bytes, void* stream)
{
    if (nseg != 1 && nseg != 2) return LKV_EINVAL;
    if (split_tokens == 0) {
        const int st = lkv_decode_plan(segs, views, nseg, batch, num_q_heads, &split_tokens);
        if (st != LKV_OK) return st;
    }
    Fmt f[2];
    const int st = check_split(segs, views, nseg, q, q_dtype, batch, num_q_heads, sm_scale, tau_low, split_tokens,
                               workspace, workspace_bytes, f);
    if (st != LKV_OK) return st;
    if (kv_dtype != LKV_F32 && kv_dtype != LKV_BF16 && kv_dtype != LKV_F16) return LKV_EINVAL;
    if (batch == 0) return LKV_OK;
    if (!k_new || !v_new || !out || !counters || (uintptr_t)counters % 4 != 0) return LKV_EINVAL;
    SegArgs a[2];
    const int32_t tot = seg_args(segs, views, nseg, f, split_tokens, nullptr, 0, 1, nullptr, 0, a);
    hipError_t e;
    const bool ok = nseg == 1
                        ? launch_append_decode_mfma(a[0], q, q_dtype, batch, num_q_heads, sm_scale, tau_low,
                                                    split_tokens, tot, (float*)workspace, k_new, v_new, kv_dtype,
                                                    (hipStream_t)stream, &e, out, counters,
                                                    ragged_hint(&views[0], batch))
                        : launch_append_decode_tiered_merged(a[0], a[1], q, q_dtype, batch, num_q_heads, sm_scale,
                                                             tau_low, split_tokens, tot, (float*)workspace, k_new,
                                                             v_new, kv_dtype, (hipStream_t)stream, &e, out,
                                                             counters);
    if (!ok) return LKV_EUNSUPPORTED;
    return e == hipSuccess ? LKV_OK : LKV_EHIP;
}

int lkv_decode_plan_multi(const lkv_cache* segs, const lkv_view* views, int32_t nseg, int32_t batch,
                          int32_t q_per_seq, int32_t num_q_heads, int32_t* split_tokens)
{
    if (q_per_seq < 1 || (int64_t)batch * q_per_seq > INT32_MAX) return LKV_EINVAL;
    // at 4 query heads per KV head the matrix-core kernel runs the query
    // tokens in pairs: plan for the work items it launches
    int32_t items = batch * q_per_seq;
    if (segs && nseg >= 1 && segs[0].num_kv_heads > 0 && num_q_heads == 4 * segs[0].num_kv_heads)
        items = batch * ((q_per_seq + 1) / 2);
    return lkv_decode_plan(segs, views, nseg, items, num_q_heads, split_tokens);
}

int lkv_decode_attn_multi(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* q,
                          int32_t q_dtype, int32_t batch, int32_t q_per_seq, int32_t num_q_heads, float sm_scale,
                          float tau_low, int32_t split_tokens, float* out, void* workspace, size_t workspace_bytes,
                          void* stream)
{
    if (q_per_seq < 1 || (int64_t)batch * q_per_seq > INT32_MAX) return LKV_EINVAL;
    const int32_t entries = batch * q_per_seq;
    for (int s = 0; s < nseg && views; s++)
        if (views[s].max_len < (s == 0 ? q_per_seq : 0) && batch > 0) return LKV_EINVAL;
    if (split_tokens == 0) {
        const int st = lkv_decode_plan_multi(segs, views, nseg, batch, q_per_seq, num_q_heads, &split_tokens);
        if (st != LKV_OK) return st;
    }
    if (batch > 0 && !out) return LKV_EINVAL;
    const int st = split_impl(segs, views, nseg, q, q_dtype, entries, num_q_heads, sm_scale, tau_low, split_tokens,
                              workspace, workspace_bytes, stream, nullptr, 0, q_per_seq);
    if (st != LKV_OK) return st;
    return combine_impl(segs, views, nseg, entries, num_q_heads, split_tokens, out, workspace, workspace_bytes, stream,
                        nullptr, false);
}

int lkv_decode_attn_debug(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* q,
                          int32_t q_dtype, int32_t batch, int32_t q_per_seq, int32_t num_q_heads, float sm_scale,
                          float tau_low, int32_t split_tokens, float* out, uint32_t* skip_mask, int32_t mask_words,
                          void* workspace, size_t workspace_bytes, void* stream)
{
    if (q_per_seq < 1 || (int64_t)batch * q_per_seq > INT32_MAX) return LKV_EINVAL;
    if (!segs || !views || nseg < 1 || nseg > 2) return LKV_EINVAL;
    for (int s = 0; s < nseg; s++)
        if (views[s].max_len < (s == 0 ? q_per_seq : 0) && batch > 0) return LKV_EINVAL;
    if (split_tokens == 0) {
        const int st = lkv_decode_plan_multi(segs, views, nseg, batch, q_per_seq, num_q_heads, &split_tokens);
        if (st != LKV_OK) return st;
    }
    const int32_t entries = batch * q_per_seq;
    Fmt f[2];
    const int st0 = check_split(segs, views, nseg, q, q_dtype, entries, num_q_heads, sm_scale, tau_low, split_tokens,
                                workspace, workspace_bytes, f);
    if (st0 != LKV_OK) return st0;
    const int64_t cols = score_cols(views, nseg);
    if (mask_words < cols / 32) return LKV_EINVAL;
    if (batch == 0) return LKV_OK;
    if (!out || !skip_mask) return LKV_EINVAL;
    const hipError_t e = launch_fill_u32(skip_mask, (int64_t)entries * num_q_heads * mask_words, 0u,
                                         (hipStream_t)stream);
    if (e != hipSuccess) return LKV_EHIP;
    const int st = split_impl(segs, views, nseg, q, q_dtype, entries, num_q_heads, sm_scale, tau_low, split_tokens,
                              workspace, workspace_bytes, stream, nullptr, 0, q_per_seq, skip_mask, mask_words);
    if (st != LKV_OK) return st;
    return combine_impl(segs, views, nseg, entries, num_q_heads, split_tokens, out, workspace, workspace_bytes, stream,
                        nullptr, false);
}

void lkv_default_thresholds(int32_t n_tokens, float* tau_low, float* tau_high)
{
    const double eps4 = 1.0 / (2.0 * 15.0);  // half a 4-bit step over the group range
    const double eps6 = 1.0 / (2.0 * 63.0);  // half a 6-bit step
    const double n = n_tokens > 0 ? (double)n_tokens : 1.0;
    if (tau_low) *tau_low = (float)(eps4 / n);
    if (tau_high) *tau_high = (float)((eps4 / eps6) / n);
}

int64_t lkv_tier_workspace_bytes(int32_t batch, int32_t scores_stride)
{
    if (batch < 0 || scores_stride < 0) return LKV_EINVAL;
    return tiering_workspace_bytes(batch, &scores_stride, 1);
}

int64_t lkv_retier_workspace_bytes(int32_t batch, int32_t h_stride, int32_t m_stride)
{
    if (batch < 0 || h_stride < 0 || m_stride < 0) return LKV_EINVAL;
    const int32_t strides[2] = {m_stride, h_stride};
    return tiering_workspace_bytes(batch, strides, 2);
}

}  // extern "C"

namespace {

// A source segment of the tiers: quantised K, vb-bit V, and the shape
// (D, g, H, K bits) of ref when ref is given.
int tier_source(const lkv_cache* c, const lkv_view* v, const float* scores, int32_t stride, uint8_t* tiers,
                int vb, int max_tier, const Fmt* ref, TierSource* out)
{
    Fmt f;
    int st = make_fmt(c, &f);
    if (st != LKV_OK) return st;
    if (f.fp16 || f.vb != vb) return ref ? LKV_EINVAL : LKV_EUNSUPPORTED;
    if (f.k_norm) return LKV_EUNSUPPORTED;  // tiers hold the plain K codec
    if (ref && (f.D != ref->D || f.g != ref->g || f.H != ref->H || f.kb != ref->kb)) return LKV_EINVAL;
    if (!v || stride < 0 || v->max_blocks < 1 || v->max_len < 0 || v->max_len > stride ||
        (int64_t)v->max_len > (int64_t)v->max_blocks * BT)
        return LKV_EINVAL;
    *out = TierSource{f, (const uint8_t*)c->pool, v->block_table, v->seq_lens, v->max_blocks, v->max_len,
                      scores, stride, tiers, max_tier};
    return LKV_OK;
}

int tier_dest(const lkv_cache* c, const int32_t* bt, int32_t max_blocks, int vb, const Fmt& ref, TierDest* out)
{
    Fmt f;
    int st = make_fmt(c, &f);
    if (st != LKV_OK) return st;
    if (f.D != ref.D || f.g != ref.g || f.H != ref.H || f.kb != ref.kb || f.vb != vb || max_blocks < 1)
        return LKV_EINVAL;
    if (f.k_norm) return LKV_EUNSUPPORTED;
    *out = TierDest{f, (uint8_t*)c->pool, bt, max_blocks};
    return LKV_OK;
}

bool sources_ready(const TierSource* s, int n)
{
    for (int i = 0; i < n; i++)
        if (!s[i].block_table || !s[i].view_lens || !s[i].scores || !s[i].tiers) return false;
    return true;
}

// A destination with a source's pool and block table is that segment
// compacted in place: only source `own` may be (-1: none), with the same
// row width.  A table shared between different pools names different blocks.
bool aliasing_ok(const TierSource* s, int nsrc, const TierDest& d, int own)
{
    for (int i = 0; i < nsrc; i++)
        if (d.pool == s[i].pool && d.block_table == s[i].block_table && (i != own || d.max_blocks != s[i].max_blocks))
            return false;
    return true;
}

}  // namespace

extern "C" {

int lkv_tier_update(const lkv_cache* src, const lkv_view* src_view, const float* scores, int32_t scores_stride,
                    float tau_low, float tau_high, const lkv_cache* dst_h, const int32_t* h_block_table,
                    int32_t h_max_blocks, const lkv_cache* dst_m, const int32_t* m_block_table,
                    int32_t m_max_blocks, int32_t* n_high, int32_t* n_mid, uint8_t* tiers, int32_t batch,
                    void* workspace, size_t workspace_bytes, void* stream)
{
    TierSource s;
    TierDest h, m;
    int st = tier_source(src, src_view, scores, scores_stride, tiers, 6, 2, nullptr, &s);
    if (st != LKV_OK) return st;
    if ((st = tier_dest(dst_h, h_block_table, h_max_blocks, 6, s.f, &h)) != LKV_OK) return st;
    if ((st = tier_dest(dst_m, m_block_table, m_max_blocks, 4, s.f, &m)) != LKV_OK) return st;
    if (batch < 0 || std::isnan(tau_low) || std::isnan(tau_high)) return LKV_EINVAL;
    if ((int64_t)workspace_bytes < lkv_tier_workspace_bytes(batch, scores_stride)) return LKV_EINVAL;
    if (batch == 0) return LKV_OK;
    if (!sources_ready(&s, 1) || !h_block_table || !m_block_table || !n_high || !n_mid || !workspace ||
        (uintptr_t)workspace % 8 != 0 || !aliasing_ok(&s, 1, h, 0) || !aliasing_ok(&s, 1, m, -1))
        return LKV_EINVAL;
    const hipError_t e = launch_tiering(&s, 1, tau_low, tau_high, h, m, n_high, n_mid, batch, workspace,
                                        (hipStream_t)stream);
    return e == hipSuccess ? LKV_OK : LKV_EHIP;
}

int lkv_retier(const lkv_cache* h, const lkv_view* h_view, const float* h_scores, int32_t h_stride,
               const lkv_cache* m, const lkv_view* m_view, const float* m_scores, int32_t m_stride,
               float tau_low, float tau_high, const lkv_cache* dst_h, const int32_t* dh_block_table,
               int32_t dh_max_blocks, const lkv_cache* dst_m, const int32_t* dm_block_table, int32_t dm_max_blocks,
               int32_t* n_high, int32_t* n_mid, uint8_t* h_tiers, uint8_t* m_tiers, int32_t batch,
               void* workspace, size_t workspace_bytes, void* stream)
{
    TierSource s[2];  // destination order: the kept MID tokens first
    TierDest dh, dm;
    int st = tier_source(h, h_view, h_scores, h_stride, h_tiers, 6, 2, nullptr, &s[1]);
    if (st != LKV_OK) return st;
    if ((st = tier_source(m, m_view, m_scores, m_stride, m_tiers, 4, 1, &s[1].f, &s[0])) != LKV_OK) return st;
    if ((st = tier_dest(dst_h, dh_block_table, dh_max_blocks, 6, s[1].f, &dh)) != LKV_OK) return st;
    if ((st = tier_dest(dst_m, dm_block_table, dm_max_blocks, 4, s[1].f, &dm)) != LKV_OK) return st;
    if (batch < 0 || std::isnan(tau_low) || std::isnan(tau_high)) return LKV_EINVAL;
    const int64_t need = lkv_retier_workspace_bytes(batch, h_stride, m_stride);
    if (need < 0 || (int64_t)workspace_bytes < need) return LKV_EINVAL;
    if (batch == 0) return LKV_OK;
    if (!sources_ready(s, 2) || !dh_block_table || !dm_block_table || !n_high || !n_mid || !workspace ||
        (uintptr_t)workspace % 8 != 0 || !aliasing_ok(s, 2, dh, 1) || !aliasing_ok(s, 2, dm, 0))
        return LKV_EINVAL;
    const hipError_t e = launch_tiering(s, 2, tau_low, tau_high, dh, dm, n_high, n_mid, batch, workspace,
                                        (hipStream_t)stream);
    return e == hipSuccess ? LKV_OK : LKV_EHIP;
}

}  // extern "C"

// ---- decode without a caller-provided workspace
//
// The split partials of lkv_decode_attn_noalloc live in this file-scope
// device array.  Every GPU the library runs on holds its own copy, at its
// own address, until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: kernels receive the address
// that hipGetSymbolAddress returns for the current device.

namespace {

static __device__ __align__(256) uint8_t scratch[LKV_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES] = {};

// Address of the current device's scratch, looked up once per device.
int scratch_of_current_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return LKV_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LKV_EHIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return LKV_OK;
}

}  // namespace

extern "C" {

int lkv_hbm_read_probe(const void* buf, int64_t bytes, int32_t nontemporal, uint32_t* sink, void* stream)
{
    if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || (uintptr_t)buf % 16 != 0) return LKV_EINVAL;
    return launch_hbm_read_probe(buf, bytes, nontemporal != 0, sink, (hipStream_t)stream) == hipSuccess ? LKV_OK
                                                                                                       : LKV_EHIP;
}

int lkv_decode_attn_noalloc(const lkv_cache* segs, const lkv_view* views, int32_t nseg, const void* q,
                            int32_t q_dtype, int32_t batch, int32_t num_q_heads, float sm_scale, float tau_low,
                            int32_t split_tokens, float* out, void* stream)
{
    if (split_tokens == 0) {
        const int st = lkv_decode_plan(segs, views, nseg, batch, num_q_heads, &split_tokens);
        if (st != LKV_OK) return st;
    }
    const int64_t need = lkv_decode_workspace_bytes(segs, views, nseg, batch, num_q_heads, split_tokens);
    if (need < 0) return (int)need;
    if (need > (int64_t)LKV_NOALLOC_SCRATCH_BYTES) return LKV_ESCRATCH;
    if (batch == 0) return LKV_OK;
    void* ws = nullptr;
    const int st = scratch_of_current_device(&ws);
    if (st != LKV_OK) return st;
    return lkv_decode_attn(segs, views, nseg, q, q_dtype, batch, num_q_heads, sm_scale, tau_low, split_tokens, out,
                           ws, (size_t)LKV_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
