// tier.hip -- attention-aware tiers (Super KV Compression page, second
// layer): the tier update of a K6V6 cache and the re-tiering of a tiered
// cache {HIGH K6V6, MID K6V4}, built with -ffp-contract=off.  One or two
// source segments, in destination order (re-tiering: MID first, so that the
// kept MID tokens come before the demoted HIGH ones).
//
//  tier_count: one workgroup per (2048-token chunk, sequence, source)
//    counts the chunk's HIGH (score >= tau_high) and MID (tau_low <= score,
//    below tau_high or from a source that is MID already) tokens.
//  tier_write: the same grid.  Each chunk adds up the counts that come
//    before it in destination order (stable), scans its own tokens, and
//    writes their tiers and the destination positions of every 64-token
//    block's first HIGH and MID survivor.  The first chunk writes the two
//    counts (negative when a destination has no room).
//  tier_compact: the survivors' rows, scales and zeros and V codes, run by
//    run (4 source chunks of one sequence, KV head and source) in
//    destination order; see the section of that name below.  A
//    destination that is its source segment itself (the same pool and
//    block table) is compacted in place: a survivor never moves to a later
//    position, so a run writes only into its own blocks or earlier ones;
//    workgroups then take their runs from a ticket counter and wait, before
//    writing into blocks that earlier workgroups own, until those blocks
//    have been read.  The sources run one launch after the other, in
//    destination order, so that the MID source's chunks are read before
//    demoted tokens land in them.
#include <hip/hip_fp16.h>

#include "lkv_internal.h"
#include "quant_device.h"

namespace lkv {

constexpr int TIER_PER = 8;  // tokens per scan thread: 256 x 8 = 2048 per workgroup
constexpr int TIER_CHUNK = 256 * TIER_PER;
static_assert(TIER_CHUNK == 2048, "tier_chunks() counts 2048-token scan chunks");

// One source segment of a scan.
struct TierSrc {
    const float* scores;
    int32_t stride;
    int32_t len_cap;
    const int32_t* lens;
    uint8_t* tiers;
    int32_t max_tier;  // 2; 1 for a source whose tokens can no longer be HIGH
    int32_t nchunks;
    int32_t chunk0;    // its first chunk in a sequence's row of counts
    int2* blk_base;    // [batch][base_stride]: (HIGH, MID) destination position of
    int32_t base_stride;  // each 64-token block's first survivor
};

struct TierScanArgs {
    TierSrc src[2];  // in destination order
    int32_t nsrc;
    float tau_low, tau_high;
    int32_t h_cap, m_cap;
    int32_t* n_high;
    int32_t* n_mid;
    int2* counts;    // [batch][count_stride] (HIGH, MID): source 0's chunks, then source 1's
    int32_t count_stride;
};

__device__ __forceinline__ int tier_of(float s, float tau_low, float tau_high, int max_tier)
{
    const int t = s >= tau_high ? 2 : (s >= tau_low ? 1 : 0);
    return min(t, max_tier);
}

// Tiers of this thread's 8 tokens of source src (3 = past the end), their
// loads issued together.
__device__ __forceinline__ void thread_tiers(const TierScanArgs& a, const TierSrc& src, int b, int len, int j0,
                                             int (&t)[TIER_PER])
{
    const float* sc = src.scores + (int64_t)b * src.stride;
    float v[TIER_PER];
#pragma unroll
    for (int i = 0; i < TIER_PER; i++) v[i] = j0 + i < len ? sc[j0 + i] : 0.0f;
#pragma unroll
    for (int i = 0; i < TIER_PER; i++)
        t[i] = j0 + i < len ? tier_of(v[i], a.tau_low, a.tau_high, src.max_tier) : 3;
}

// Sum over the 256-thread workgroup of (h, m), every thread gets the total.
__device__ __forceinline__ int2 block_sum2(int h, int m, int2* red)
{
    for (int o = 32; o > 0; o >>= 1) {
        h += __shfl_xor(h, o, 64);
        m += __shfl_xor(m, o, 64);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = make_int2(h, m);
    __syncthreads();
    int2 r = make_int2(0, 0);
#pragma unroll
    for (int w = 0; w < 4; w++) { r.x += red[w].x; r.y += red[w].y; }
    return r;
}

// grid (chunks, batch, sources)
__global__ __launch_bounds__(256) void tier_count_kernel(TierScanArgs a)
{
    const int c = blockIdx.x, b = blockIdx.y;
    const TierSrc& src = blockIdx.z == 0 ? a.src[0] : a.src[1];
    if (c >= src.nchunks) return;
    const int len = max(0, min(src.lens[b], src.len_cap));  // out-of-contract lengths are clamped
    const int j0 = c * TIER_CHUNK + TIER_PER * threadIdx.x;
    int t[TIER_PER];
    thread_tiers(a, src, b, len, j0, t);
    int h = 0, m = 0;
#pragma unroll
    for (int i = 0; i < TIER_PER; i++) {
        h += t[i] == 2;
        m += t[i] == 1;
    }
    __shared__ int2 red[4];
    const int2 r = block_sum2(h, m, red);
    if (threadIdx.x == 0) a.counts[(int64_t)b * a.count_stride + src.chunk0 + c] = r;
}

__global__ __launch_bounds__(256) void tier_write_kernel(TierScanArgs a)
{
    const int c = blockIdx.x, b = blockIdx.y, z = blockIdx.z;
    const TierSrc& src = z == 0 ? a.src[0] : a.src[1];
    if (c >= src.nchunks) return;
    const int len = max(0, min(src.lens[b], src.len_cap));
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // totals over every source, and the counts that come before this chunk
    // in destination order (earlier sources, then earlier chunks)
    const int self = src.chunk0 + c;
    int th = 0, tm = 0, bh = 0, bm = 0;
    for (int i = lane; i < a.count_stride; i += 64) {
        const int2 v = a.counts[(int64_t)b * a.count_stride + i];
        th += v.x;
        tm += v.y;
        if (i < self) { bh += v.x; bm += v.y; }
    }
    for (int o = 32; o > 0; o >>= 1) {
        th += __shfl_xor(th, o, 64);
        tm += __shfl_xor(tm, o, 64);
        bh += __shfl_xor(bh, o, 64);
        bm += __shfl_xor(bm, o, 64);
    }
    const bool fits = th <= a.h_cap && tm <= a.m_cap;
    if (z == 0 && c == 0 && tid == 0) {
        a.n_high[b] = fits ? th : -th;
        a.n_mid[b] = fits ? tm : -tm;
    }
    const int j0 = c * TIER_CHUNK + TIER_PER * tid;
    int t[TIER_PER];
    thread_tiers(a, src, b, len, j0, t);
    uint8_t* tr = src.tiers + (int64_t)b * src.stride;
#pragma unroll
    for (int i = 0; i < TIER_PER; i++)
        if (t[i] < 3) tr[j0 + i] = (uint8_t)t[i];
    if (!fits) return;
    int ch = 0, cm = 0;
#pragma unroll
    for (int i = 0; i < TIER_PER; i++) {
        ch += t[i] == 2;
        cm += t[i] == 1;
    }
    // exclusive scan of (ch, cm) over the workgroup
    int ih = ch, im = cm;
    for (int o = 1; o < 64; o <<= 1) {
        const int uh = __shfl_up(ih, o, 64), um = __shfl_up(im, o, 64);
        if (lane >= o) { ih += uh; im += um; }
    }
    __shared__ int2 wsum[4];
    if (lane == 63) wsum[wave] = make_int2(ih, im);
    __syncthreads();
    int ph = bh + ih - ch, pm = bm + im - cm;
    for (int w = 0; w < wave; w++) { ph += wsum[w].x; pm += wsum[w].y; }
    // eight threads hold one 64-token block: the first writes its base
    static_assert(8 * TIER_PER == BT, "a block is eight scan threads");
    if ((tid & 7) == 0 && j0 < len) src.blk_base[(int64_t)b * src.base_stride + j0 / BT] = make_int2(ph, pm);
}

struct MoveSrc {
    Fmt f;
    const uint8_t* pool;
    const int32_t* bt;
    int32_t max_blocks;
    const int32_t* lens;
    int32_t len_cap;
    const uint8_t* tiers;
    int32_t tier_stride;
    const int2* blk_base;
    int32_t base_stride;
};

struct MoveDst {
    Fmt f;
    uint8_t* pool;
    const int32_t* bt;
    int32_t max_blocks;
};

struct MoveArgs {
    MoveSrc src[2];
    MoveDst dst[2];  // 0: HIGH, 1: MID
    const int32_t* n_high;
    const int32_t* n_mid;
    int32_t nsrc;
    int32_t per_wg;  // runs per workgroup
    // in place: one source; a workgroup's (sequence, group of runs, KV head)
    // comes from *ticket; flags[b][run] counts the KV heads that have read
    // a run's chunks; inplace_seg is the destination (0 HIGH, 1 MID) that
    // is the source
    uint32_t* ticket;
    uint32_t* flags;
    int32_t flag_stride;
    int32_t inplace_seg;
    int32_t gx;      // groups of runs per sequence in the ticket order
};

// ---- Compaction: tier_compact_kernel<D, g, in place> ----
//
// One workgroup per run of CMP_R consecutive source chunks of one
// (sequence, KV head, source); wave w owns chunk w of the run.
//  1. The run's V sections are loaded (coalesced, 16 B per thread) while
//     each wave moves its chunk's K rows, K scales and zeros, and the V
//     scales and zeros of survivors whose V codes are copied: lane = slot,
//     every survivor's row goes straight from its source slot to its
//     destination slot.  Nothing of an evicted token is read.
//  2. The V sections go to LDS and the survivors of the run are listed per
//     destination segment, in slot order (ranks).
//  3. V codes are written per window of TPW destination slots (aligned, so
//     a window's words hold no slot of another window): lane = (slot of the
//     window, half of the channels).  Each lane takes its survivor's codes
//     from LDS, copies them or requantises them at 4 bits (the group's
//     extremes from the extreme codes, since the dequantised value is
//     monotone in the code; every lane holds whole groups, so no lane
//     exchange), and puts them in a small per-wave stage from which whole
//     words are packed and stored.  Words that also hold slots of a
//     neighbouring run are merged with atomics.
constexpr int CMP_R = 4;  // source chunks per run (one per wave)
constexpr int CMP_S = 8;  // most runs per workgroup, one after the other (MoveArgs::per_wg)
typedef uint32_t cmp_u32x4 __attribute__((ext_vector_type(4)));

// Orders one wave's LDS stores before its later LDS loads (other lanes).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Step 1 for one survivor (lane) of segment SEG (0 HIGH, 1 MID); P its
// destination position.  KR 16-byte pieces per K row, NG quantisation
// groups.  Every load is issued before the first store.
template <int KR, int NG, int SEG>
__device__ __forceinline__ void compact_row(const MoveArgs& a, const Fmt& fs, const uint8_t* sch, int P, int b,
                                            int kvh, int lane, bool vcopy)
{
    const MoveDst& d = a.dst[SEG];
    const int32_t blk = d.bt[(int64_t)b * d.max_blocks + P / BT];
    const cmp_u32x4* ks = (const cmp_u32x4*)(sch + fs.off_kc + lane * (16 * KR));
    cmp_u32x4 kv[KR];
#pragma unroll
    for (int i = 0; i < KR; i++) kv[i] = ks[i];
    float k_s[NG], v_s[NG];
    uint32_t k_z[NG], v_z[NG];
#pragma unroll
    for (int gi = 0; gi < NG; gi++) {
        k_s[gi] = ((const float*)(sch + fs.off_ks))[gi * BT + lane];
        k_z[gi] = sch[fs.off_kz + gi * BT + lane];
        if (vcopy) {
            v_s[gi] = ((const float*)(sch + fs.off_vs))[gi * BT + lane];
            v_z[gi] = sch[fs.off_vz + gi * BT + lane];
        }
    }
    uint8_t* dch = d.pool + ((int64_t)blk * fs.H + kvh) * d.f.chunk;
    const int ds = P % BT;
    cmp_u32x4* kd = (cmp_u32x4*)(dch + d.f.off_kc + ds * (16 * KR));
#pragma unroll
    for (int i = 0; i < KR; i++) kd[i] = kv[i];
#pragma unroll
    for (int gi = 0; gi < NG; gi++) {
        ((float*)(dch + d.f.off_ks))[gi * BT + ds] = k_s[gi];
        dch[d.f.off_kz + gi * BT + ds] = (uint8_t)k_z[gi];
        if (vcopy) {
            ((float*)(dch + d.f.off_vs))[gi * BT + ds] = v_s[gi];
            dch[d.f.off_vz + gi * BT + ds] = (uint8_t)v_z[gi];
        }
    }
}

template <int D, int NG, int SEG>
__device__ __forceinline__ void compact_row_any(const MoveArgs& a, const Fmt& fs, const uint8_t* sch, int P, int b,
                                                int kvh, int lane, bool vcopy)
{
    constexpr int K4 = D / 32, K6 = D * 6 / 128;  // 16-byte pieces of a 4- or 6-bit K row
    if (fs.kb == 6) compact_row<K6, NG, SEG>(a, fs, sch, P, b, kvh, lane, vcopy);
    else compact_row<K4, NG, SEG>(a, fs, sch, P, b, kvh, lane, vcopy);
}

template <int D, int NG, bool IP = false>
struct alignas(16) CmpShared {
    static constexpr int NH = D / 64;          // channel halves: lanes per survivor
    static constexpr int TPW = 64 / NH;        // destination slots per window
    static constexpr int CW = D * 12 + 4;      // words per staged V section (6-bit rows; 4-bit use less)
    static constexpr int SP = TPW + 16;        // stage row pitch (bytes, a multiple of 16)
    // in place (IP) whole source chunks, so that a run has read everything
    // before it marks its chunks read; otherwise only the V sections and,
    // for requantised MID survivors, the V scales and zeros
    static constexpr int IMG = (96 * D + 10 * NG * BT + 15) / 16 * 16;  // the largest chunk (K6V6)
    uint8_t img[IP ? CMP_R : 1][IP ? IMG : 16];
    uint32_t vsec[IP ? 1 : CMP_R][IP ? 1 : CW];
    float vs[IP ? 1 : CMP_R][IP ? 1 : NG * BT];
    uint8_t vz[IP ? 1 : CMP_R][IP ? 1 : NG * BT];
    uint8_t stage[4][16 * NH][SP];             // per wave: 16 channels of each half x TPW slots
    uint16_t lst[2][CMP_R * BT];               // survivors per segment: (chunk of the run << 6) | slot
    int32_t cnt[2][CMP_R];
    int32_t dblk[2][8];                        // destination blocks from the run's first position
    // a segment's last word when the run ends inside it, carried into the
    // workgroup's next run: [run parity][segment], and {valid, low bit,
    // high bit, word, destination block}
    uint32_t carry[2][2][D];
    int32_t cmeta[2][2][8];

    __device__ __forceinline__ const uint32_t* vrows(int cl, const Fmt& fs) const
    {
        if constexpr (IP) return (const uint32_t*)(img[cl] + fs.off_vc);
        else return vsec[cl];
    }
    __device__ __forceinline__ float vscale(int cl, const Fmt& fs, int i) const
    {
        if constexpr (IP) return ((const float*)(img[cl] + fs.off_vs))[i];
        else return vs[cl][i];
    }
    __device__ __forceinline__ int vzero(int cl, const Fmt& fs, int i) const
    {
        if constexpr (IP) return img[cl][fs.off_vz + i];
        else return vz[cl][i];
    }
};

// Where a window's words go: the destination chunk, the run's slots [lo, hi)
// relative to that chunk's block, and the carries in and out.
struct WordSink {
    uint8_t* dch;
    int off_vc, vrow, lo, hi, blk;
    const uint32_t* cin;    // the word the previous run ended inside, or null
    int cin_lo;
    uint32_t* cout;
    int32_t* cmeta_out;
};

// Word W of channel row d holds this run's bits [a, e) (e > a).  A word the
// run completes is stored whole (with the carried bits of the previous run
// when it starts inside the word); one the run ends inside is carried; one
// that starts with another workgroup's bits is merged with atomics.
template <int NB>
__device__ __forceinline__ void sink_word(const WordSink& k, int d, int W, uint32_t w)
{
    const int a = min(32, max(0, NB * k.lo - 32 * W)), e = min(32, max(0, NB * k.hi - 32 * W));
    if (e <= a) return;
    const uint32_t top = e == 32 ? 0xFFFFFFFFu : ((1u << e) - 1u);
    uint32_t val = w & (top & ~((1u << a) - 1u));
    int low = a;
    if (a > 0 && k.cin) {
        val |= k.cin[d];
        low = k.cin_lo;
    }
    if (e < 32) {
        k.cout[d] = val;
        if (d == 0) {
            k.cmeta_out[0] = 1;
            k.cmeta_out[1] = low;
            k.cmeta_out[2] = e;
            k.cmeta_out[3] = W;
            k.cmeta_out[4] = k.blk;
        }
        return;
    }
    uint32_t* p = (uint32_t*)(k.dch + k.off_vc + d * k.vrow) + W;
    if (low == 0) {
        *p = val;
    } else {
        atomicAnd(p, (1u << low) - 1u);
        atomicOr(p, val);
    }
}

// Code of channel row dl (of the lane's half) at slot s of a staged section.
template <int VB>
__device__ __forceinline__ uint32_t staged_code(const uint32_t* row, int dl, int ws, int sh)
{
    constexpr int VW = 2 * VB;  // words per row: 64 slots x VB bits
    if constexpr (VB == 6) {
        return __builtin_amdgcn_alignbit(row[dl * VW + ws + 1], row[dl * VW + ws], sh) & 63u;
    } else {
        return (row[dl * VW + ws] >> sh) & 15u;
    }
}

// Packs the wave's stage (16 channels of each half, block jb of the
// channel loop) into NB-bit words of destination chunk dch, window k; only
// fields of slots [lo, hi) (relative to the window's block) are written.
template <int D, int NB>
__device__ __forceinline__ void pack_stage(const uint8_t (*st)[CmpShared<D, 1>::SP], const WordSink& sink, int k,
                                           int jb, int lane)
{
    constexpr int NH = CmpShared<D, 1>::NH, TPW = CmpShared<D, 1>::TPW;
    constexpr int FPG = NB == 4 ? 8 : 16;  // fields per packed group
    constexpr int GPR = TPW / FPG;
    constexpr int ITEMS = 16 * NH * GPR;
    const int s0 = (k * TPW) % BT;  // the window's first slot in its block
#pragma unroll
    for (int it = 0; it < (ITEMS + 63) / 64; it++) {
        const int idx = lane + 64 * it;
        if (ITEMS % 64 != 0 && idx >= ITEMS) break;
        const int i = idx / GPR, gq = idx % GPR;
        const int d = 64 * (i / 16) + 16 * jb + (i % 16);
        const int slot = s0 + gq * FPG;
        if constexpr (NB == 4) {
            const uint2 x = *(const uint2*)(st[i] + gq * FPG);
            const uint32_t yl = x.x | (x.x >> 4), yh = x.y | (x.y >> 4);
            const uint32_t w = (yl & 0xFFu) | ((yl >> 8) & 0xFF00u) | ((yh & 0xFFu) << 16) | ((yh << 8) & 0xFF000000u);
            sink_word<4>(sink, d, slot / 8, w);
        } else {
            const uint4 x = *(const uint4*)(st[i] + gq * FPG);
            uint32_t v[16], w[3];
            const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int q = 0; q < 4; q++) {
                v[4 * q] = xs[q] & 0xFFu;
                v[4 * q + 1] = (xs[q] >> 8) & 0xFFu;
                v[4 * q + 2] = (xs[q] >> 16) & 0xFFu;
                v[4 * q + 3] = xs[q] >> 24;
            }
            pack_values<6, 16, 3>(v, w);
            const int W0 = slot / 16 * 3;
#pragma unroll
            for (int q = 0; q < 3; q++) sink_word<6>(sink, d, W0 + q, w[q]);
        }
    }
}

// One window of copied codes (VB bits at the source and the destination).
template <int D, int NG, int VB, bool IP>
__device__ __forceinline__ void compact_copy(CmpShared<D, NG, IP>& sh, const Fmt& fs, const MoveDst& dst, int kvh,
                                             int seg, int k, int plo, int n, int wave, int lane, WordSink sink)
{
    constexpr int NH = CmpShared<D, NG>::NH, TPW = CmpShared<D, NG>::TPW;
    const int t = lane % TPW, h = lane / TPW;
    const int p = k * TPW + t, r = p - plo;
    const bool valid = r >= 0 && r < n;
    const int e = sh.lst[seg][valid ? r : 0];
    const int cl = e >> 6, s = e & 63;
    const uint32_t* row = sh.vrows(cl, fs) + 64 * h * (2 * VB);
    const int bit = s * VB, ws = bit >> 5, bsh = bit & 31;
    const int blk0 = k * TPW / BT * BT;
    sink.blk = sh.dblk[seg][blk0 / BT - plo / BT];
    sink.dch = dst.pool + ((int64_t)sink.blk * dst.f.H + kvh) * dst.f.chunk;
    sink.off_vc = dst.f.off_vc;
    sink.vrow = dst.f.vrow;
    sink.lo = plo - blk0;
    sink.hi = plo + n - blk0;
    auto st = sh.stage[wave];
    for (int jb = 0; jb < 4; jb++) {
        // all 16 loads first: the stage stores could alias them for the compiler
        uint32_t code[16];
#pragma unroll
        for (int j = 0; j < 16; j++) code[j] = staged_code<VB>(row, 16 * jb + j, ws, bsh);
#pragma unroll
        for (int j = 0; j < 16; j++) st[h * 16 + j][t] = (uint8_t)code[j];
        wave_lds_sync();
        pack_stage<D, VB>(st, sink, k, jb, lane);
        wave_lds_sync();
    }
    (void)NH;
}

// One window of MID codes requantised from 6 to 4 bits, with their V scales
// and zeros; groups of GS channels.  The same codes, scales and zero points
// as quantize_fast / quantize_exact over the dequantised row: the group's
// min / max are the dequantised extreme codes; a quotient that the fast
// division leaves uncertain is recomputed with correctly rounded division.
template <int D, int GS, bool IP>
__device__ __forceinline__ void compact_requant(CmpShared<D, D / GS, IP>& sh, const Fmt& fs, const MoveArgs& a, int kvh,
                                                int k, int plo, int n, int wave, int lane, WordSink sink)
{
    constexpr int TPW = CmpShared<D, D / GS>::TPW, GL = 64 / GS;
    const MoveDst& dst = a.dst[1];
    const Fmt& fm = dst.f;
    const int t = lane % TPW, h = lane / TPW;
    const int p = k * TPW + t, r = p - plo;
    const bool valid = r >= 0 && r < n;
    const int e = sh.lst[1][valid ? r : 0];
    const int cl = e >> 6, s = e & 63;
    float sv[GL];
    int zv[GL];
#pragma unroll
    for (int gl = 0; gl < GL; gl++) {
        const int gi = h * GL + gl;
        sv[gl] = sh.vscale(cl, fs, gi * BT + s);
        zv[gl] = sh.vzero(cl, fs, gi * BT + s);
    }
    const uint32_t* row = sh.vrows(cl, fs) + 64 * h * 12;
    const int bit = s * 6, ws = bit >> 5, bsh = bit & 31;
    int cmn[GL], cmx[GL];
#pragma unroll
    for (int gl = 0; gl < GL; gl++) { cmn[gl] = 63; cmx[gl] = 0; }
#pragma unroll
    for (int j = 0; j < 64; j++) {
        const int c = (int)staged_code<6>(row, j, ws, bsh);
        cmn[j / GS] = min(cmn[j / GS], c);
        cmx[j / GS] = max(cmx[j / GS], c);
    }
    float qs[GL], qrc[GL];
    int qz[GL], cq[GL];
    bool gslow[GL], cst[GL];
    {
#pragma clang fp contract(off)
#pragma unroll
        for (int gl = 0; gl < GL; gl++) {
            const float xa = (float)(cmn[gl] - zv[gl]) * sv[gl];
            const float xb = (float)(cmx[gl] - zv[gl]) * sv[gl];
            const int ka = fkey(xa), kb = fkey(xb);
            const float mn = fkey_value(min(ka, kb)), mx = fkey_value(max(ka, kb));
            const float lo = mn < 0.0f ? mn : 0.0f;
            const float hi = mx > 0.0f ? mx : 0.0f;
            const float rr = hi - lo;
            const float s0 = rr * 0x1.111112p-4f;  // RN(1/15)
            const float sc = __builtin_fmaf(__builtin_fmaf(-s0, 15.0f, rr), 0x1.111112p-4f, s0);
            const float rc = __builtin_amdgcn_rcpf(sc);
            bool slow = !(sc >= 0x1p-126f && sc <= 0x1.fffffep127f);
            float zf = slow ? 0.0f : rint_quot(-lo, sc, rc, slow);
            if (slow) zf = rintf(-lo / sc);
            int z = (int)zf;
            z = z < 0 ? 0 : (z > 15 ? 15 : z);
            qs[gl] = sc;
            qrc[gl] = rc;
            qz[gl] = z;
            gslow[gl] = !(sc >= 0x1p-126f && sc <= 0x1.fffffep127f);
            cst[gl] = mn == mx;
            cq[gl] = mn > 0.0f ? 1 : 0;
            if (cst[gl]) {
                qs[gl] = mn > 0.0f ? mn : (mn < 0.0f ? -mn : 0.0f);
                qz[gl] = mn < 0.0f ? 1 : 0;
            }
        }
    }
    const int blk0 = k * TPW / BT * BT;
    sink.blk = sh.dblk[1][blk0 / BT - plo / BT];
    uint8_t* dch = dst.pool + ((int64_t)sink.blk * fm.H + kvh) * fm.chunk;
    sink.dch = dch;
    sink.off_vc = fm.off_vc;
    sink.vrow = fm.vrow;
    sink.lo = plo - blk0;
    sink.hi = plo + n - blk0;
    if (valid) {
        const int ds = p % BT;
#pragma unroll
        for (int gl = 0; gl < GL; gl++) {
            const int gi = h * GL + gl;
            ((float*)(dch + fm.off_vs))[gi * BT + ds] = qs[gl];
            dch[fm.off_vz + gi * BT + ds] = (uint8_t)qz[gl];
        }
    }
    auto st = sh.stage[wave];
    for (int jb = 0; jb < 4; jb++) {
        int code[16];
#pragma unroll
        for (int j = 0; j < 16; j++) code[j] = (int)staged_code<6>(row, 16 * jb + j, ws, bsh);
#pragma unroll
        for (int j = 0; j < 16; j++) {
#pragma clang fp contract(off)
            const int jj = 16 * jb + j, gl = jj / GS;
            const int c = code[j];
            const float x = (float)(c - zv[gl]) * sv[gl];
            bool slow = gslow[gl];
            float qf = rint_quot(x, qs[gl], qrc[gl], slow);
            if (slow) qf = rintf(x / qs[gl]);
            int q = (int)qf + qz[gl];
            q = q < 0 ? 0 : (q > 15 ? 15 : q);
            st[h * 16 + j][t] = (uint8_t)(cst[gl] ? cq[gl] : q);
        }
        wave_lds_sync();
        pack_stage<D, 4>(st, sink, k, jb, lane);
        wave_lds_sync();
    }
}

template <int D, int GS, int VS, bool IP>
__device__ __forceinline__ void tier_compact_body(CmpShared<D, D / GS, IP>& sh, const MoveArgs& a, const MoveSrc& S,
                                                  int b, int kvh, int len, int c0, int nc, int par, int cwg)
{
    constexpr int NG = D / GS;
    const Fmt& fs = S.f;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t* brow = S.bt + (int64_t)b * S.max_blocks;
    const bool copy_m = a.dst[1].f.vb == VS;
    const bool requant = VS == 6 && !copy_m;
    typedef __attribute__((address_space(1))) void gvoid;
    typedef __attribute__((address_space(3))) void lvoid;

    // 1. each wave's chunk: its V section (and, when MID survivors are
    //    requantised, its V scales and zeros; in place the whole chunk)
    //    copied into LDS by the memory unit, its rows moved by the lanes
    //    (in place only after step 2).  Everything the windows read from
    //    memory is staged here, before the barrier.
    constexpr int NPC = D * VS * 64 / 8 / 16;  // 16-byte pieces of a V section
    static_assert(NPC % 64 == 0, "whole wave copies");
    const bool live = wave < nc;
    const int c = c0 + min(wave, nc - 1);
    const int tok = c * BT + lane;
    const int traw = S.tiers[(int64_t)b * S.tier_stride + min(tok, len - 1)];
    const int2 base_c = S.blk_base[(int64_t)b * S.base_stride + c];
    const int2 base = S.blk_base[(int64_t)b * S.base_stride + c0];
    const int32_t blk_c = brow[c];
    if (tid < 16) {  // destination blocks of each segment from the run's first position on
        const int seg = tid / 8;
        const MoveDst& d = seg == 0 ? a.dst[0] : a.dst[1];
        const int first = (seg == 0 ? base.x : base.y) / BT;
        sh.dblk[seg][tid % 8] = d.bt[(int64_t)b * d.max_blocks + min(first + tid % 8, d.max_blocks - 1)];
    }
    const uint8_t* sch = S.pool + ((int64_t)blk_c * fs.H + kvh) * fs.chunk;
    if (live) {
        if constexpr (IP) {
            constexpr int NI = (CmpShared<D, NG, IP>::IMG + 1023) / 1024;
#pragma unroll
            for (int i = 0; i < NI; i++)
                if (16 * (64 * i + lane) < fs.chunk)
                    __builtin_amdgcn_global_load_lds((gvoid*)(sch + 16 * (64 * i + lane)),
                                                     (lvoid*)(sh.img[wave] + 1024 * i), 16, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < NPC / 64; i++)
                __builtin_amdgcn_global_load_lds((gvoid*)(sch + fs.off_vc + 16 * (64 * i + lane)),
                                                 (lvoid*)((uint8_t*)sh.vsec[wave] + 1024 * i), 16, 0, 0);
            if (requant) {
                if (lane < NG * 16)
                    __builtin_amdgcn_global_load_lds((gvoid*)(sch + fs.off_vs + 16 * lane), (lvoid*)sh.vs[wave], 16,
                                                     0, 0);
                if (lane < NG * 4)
                    __builtin_amdgcn_global_load_lds((gvoid*)(sch + fs.off_vz + 16 * lane), (lvoid*)sh.vz[wave], 16,
                                                     0, 0);
            }
        }
    }
    const int tw = live && tok < len ? traw : 0;
    const uint64_t mk0 = __ballot(tw == 2), mk1 = __ballot(tw == 1);
    const uint64_t below = (1ull << lane) - 1ull;
    const int r0 = __popcll(mk0 & below), r1 = __popcll(mk1 & below);
    if (lane == 0) {
        sh.cnt[0][wave] = __popcll(mk0);
        sh.cnt[1][wave] = __popcll(mk1);
    }
    if (tid < 2) sh.cmeta[par][tid][0] = 0;  // nothing carried out yet (this parity was read by the run before last)
    if constexpr (!IP) {
        if (mk0 && tw == 2) compact_row_any<D, NG, 0>(a, fs, sch, base_c.x + r0, b, kvh, lane, true);
        if (mk1 && tw == 1) compact_row_any<D, NG, 1>(a, fs, sch, base_c.y + r1, b, kvh, lane, copy_m);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the sections are in LDS
    __syncthreads();

    // 2. survivors of the run per segment, in slot order
    int pre0 = 0, pre1 = 0, n0 = 0, n1 = 0;
#pragma unroll
    for (int w = 0; w < CMP_R; w++) {
        const int x0 = sh.cnt[0][w], x1 = sh.cnt[1][w];
        if (w < wave) { pre0 += x0; pre1 += x1; }
        n0 += x0;
        n1 += x1;
    }
    if (tw == 2) sh.lst[0][pre0 + r0] = (uint16_t)((wave << 6) | lane);
    else if (tw == 1) sh.lst[1][pre1 + r1] = (uint16_t)((wave << 6) | lane);
    if constexpr (IP) {
        // The run's chunks are read (every load has returned): mark them for
        // this KV head.  Then wait until the blocks the run writes into that
        // belong to earlier workgroups (below cwg, the workgroup's first
        // chunk) have been read by every KV head: those workgroups hold
        // earlier tickets and mark each run before they wait for anything.
        // Relaxed device-scope atomics: the order needed is a load's return
        // before another workgroup's store to the same bytes.
        uint32_t* frow = a.flags + (int64_t)b * a.flag_stride;
        if (tid == 0) __hip_atomic_fetch_add(frow + c0 / CMP_R, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int own = a.inplace_seg;
        const int n_own = own == 0 ? n0 : n1, p_own = own == 0 ? base.x : base.y;
        if (n_own > 0) {
            const int jlo = p_own / BT / CMP_R, jhi = min((p_own + n_own - 1) / BT, cwg - 1) / CMP_R;
            const uint32_t heads = (uint32_t)fs.H;
            if (p_own / BT < cwg)
                for (int j = jlo + tid; j <= jhi; j += 256)
                    for (uint32_t spin = 0; spin < (1u << 20); spin++) {
                        if (__hip_atomic_load(frow + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= heads) break;
                        __builtin_amdgcn_s_sleep(2);
                    }
        }
    }
    __syncthreads();
    if constexpr (IP) {
        const uint8_t* img = (const uint8_t*)sh.img[wave];
        if (mk0 && tw == 2) compact_row_any<D, NG, 0>(a, fs, img, base_c.x + r0, b, kvh, lane, true);
        if (mk1 && tw == 1) compact_row_any<D, NG, 1>(a, fs, img, base_c.y + r1, b, kvh, lane, copy_m);
    }

    // 3. windows of destination slots: MID first (the costlier ones), then HIGH
    constexpr int TPW = CmpShared<D, NG>::TPW;
    const int win0 = n0 ? (base.x + n0 - 1) / TPW - base.x / TPW + 1 : 0;
    const int win1 = n1 ? (base.y + n1 - 1) / TPW - base.y / TPW + 1 : 0;
    WordSink sk[2];
#pragma unroll
    for (int seg = 0; seg < 2; seg++) {
        sk[seg].cin = sh.cmeta[par ^ 1][seg][0] ? sh.carry[par ^ 1][seg] : nullptr;
        sk[seg].cin_lo = sh.cmeta[par ^ 1][seg][1];
        sk[seg].cout = sh.carry[par][seg];
        sk[seg].cmeta_out = sh.cmeta[par][seg];
    }
    for (int q = wave; q < win0 + win1; q += 4) {
        if (q < win1) {
            const int k = base.y / TPW + q;
            if (VS == 4) compact_copy<D, NG, 4, IP>(sh, fs, a.dst[1], kvh, 1, k, base.y, n1, wave, lane, sk[1]);
            else compact_requant<D, GS, IP>(sh, fs, a, kvh, k, base.y, n1, wave, lane, sk[1]);
        } else if (VS == 6) {
            const int k = base.x / TPW + q - win1;
            compact_copy<D, NG, 6, IP>(sh, fs, a.dst[0], kvh, 0, k, base.x, n0, wave, lane, sk[0]);
        }
    }
    __syncthreads();
    // a segment without survivors in this run passes its carry on
#pragma unroll
    for (int seg = 0; seg < 2; seg++) {
        if ((seg == 0 ? n0 : n1) != 0) continue;
        for (int d = tid; d < D; d += 256) sh.carry[par][seg][d] = sh.carry[par ^ 1][seg][d];
        if (tid < 8) sh.cmeta[par][seg][tid] = sh.cmeta[par ^ 1][seg][tid];
    }
}

// Out of place: grid (groups of per_wg runs of CMP_R chunks, KV heads,
// batch x sources).  In place (IP, one source per launch): a 1-D grid whose
// workgroups take their (sequence, group, KV head) from a ticket counter,
// a sequence's groups in order and their KV heads together; flags[b][run]
// counts the KV heads that have read a run.  256 threads; GS channels per
// quantisation group.  Sources are 6-bit (HIGH copied, MID requantised) or
// 4-bit (MID copied).
template <int D, int GS, bool IP>
__device__ __forceinline__ void tier_compact(const MoveArgs& a)
{
    __shared__ CmpShared<D, D / GS, IP> sh;
    __shared__ int ticket_of;
    int si, b, kvh, g;
    if constexpr (IP) {  // every workgroup takes a ticket before anything else
        if (threadIdx.x == 0) ticket_of = (int)atomicAdd(a.ticket, 1u);
        __syncthreads();
        const int t = ticket_of, H = a.src[0].f.H;
        si = 0;
        kvh = t % H;
        g = t / H % a.gx;
        b = t / H / a.gx;
    } else {
        si = blockIdx.z % a.nsrc;
        b = blockIdx.z / a.nsrc;
        kvh = blockIdx.y;
        g = blockIdx.x;
    }
    if (a.n_high[b] < 0 || a.n_mid[b] < 0) return;  // no room: nothing is written
    const MoveSrc& S = si == 0 ? a.src[0] : a.src[1];
    const int len = max(0, min(S.lens[b], S.len_cap));
    const int nblocks = (len + BT - 1) / BT;
    const int S_ = a.per_wg;
    const int cwg = g * S_ * CMP_R;
    if (cwg >= nblocks) return;
    if (threadIdx.x < 4) sh.cmeta[threadIdx.x / 2][threadIdx.x % 2][0] = 0;
    const int runs = min(S_, (nblocks - cwg + CMP_R - 1) / CMP_R);
    auto each_run = [&](auto vs) __attribute__((always_inline)) {
#pragma nounroll
        for (int r = 0; r < runs; r++) {
            const int c0 = cwg + r * CMP_R;
            tier_compact_body<D, GS, decltype(vs)::value, IP>(sh, a, S, b, kvh, len, c0, min(CMP_R, nblocks - c0),
                                                              r & 1, cwg);
            __syncthreads();
        }
    };
    if (S.f.vb == 6) each_run(std::integral_constant<int, 6>());
    else each_run(std::integral_constant<int, 4>());
    // the words the last runs ended inside: merged with the neighbours' bits
    const int par = (runs - 1) & 1;
#pragma unroll
    for (int seg = 0; seg < 2; seg++) {
        const int32_t* m = sh.cmeta[par][seg];
        if (!m[0]) continue;
        const MoveDst& d = seg == 0 ? a.dst[0] : a.dst[1];
        const uint32_t mask = (m[2] == 32 ? 0xFFFFFFFFu : ((1u << m[2]) - 1u)) & ~((1u << m[1]) - 1u);
        uint8_t* dch = d.pool + ((int64_t)m[4] * d.f.H + kvh) * d.f.chunk + d.f.off_vc;
        for (int ch = threadIdx.x; ch < D; ch += 256) {
            uint32_t* p = (uint32_t*)(dch + ch * d.f.vrow) + m[3];
            atomicAnd(p, ~mask);
            atomicOr(p, sh.carry[par][seg][ch] & mask);
        }
    }
}

// Four waves per SIMD for groups of 32 or 64 channels (at most 128
// registers); groups of 16 need more registers than that.
template <int D, int GS, bool IP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void tier_compact_kernel(MoveArgs a)
{
    tier_compact<D, GS, IP>(a);
}

// In place: whole chunks in LDS allow two workgroups per compute unit, so
// no register cap.
template <int D, int GS>
__global__ __launch_bounds__(256) void tier_compact_ip_kernel(MoveArgs a)
{
    tier_compact<D, GS, true>(a);
}

template <int D>
__global__ __launch_bounds__(256) void tier_compact16_kernel(MoveArgs a)
{
    tier_compact<D, 16, false>(a);
}

hipError_t launch_tiering(const TierSource* src, int nsrc, float tau_low, float tau_high, const TierDest& h,
                          const TierDest& m, int32_t* n_high, int32_t* n_mid, int32_t batch, void* workspace,
                          hipStream_t stream)
{
    if (batch == 0) return hipSuccess;
    for (int i = 0; i < nsrc; i++)  // every quantised format (K and V at 4 or 6 bits) fits the staging
        if (src[i].f.kb > 6 || src[i].f.vb > 6 || src[i].f.D != h.f.D || src[i].f.g != h.f.g)
            return hipErrorInvalidValue;
    TierScanArgs t = {};
    int2* counts = (int2*)workspace;
    int32_t count_stride = 0, base_total = 0, max_chunks = 0, max_blocks = 0;
    for (int i = 0; i < nsrc; i++) {
        count_stride += tier_chunks(src[i].stride);
        max_blocks = max(max_blocks, (src[i].max_len + BT - 1) / BT);
    }
    int2* bases = counts + (int64_t)batch * count_stride;
    for (int i = 0; i < nsrc; i++) {
        TierSrc& s = t.src[i];
        s.scores = src[i].scores;
        s.stride = src[i].stride;
        s.len_cap = src[i].max_len;  // lengths above max_len read as max_len (max_len <= stride, validated)
        s.lens = src[i].view_lens;
        s.tiers = src[i].tiers;
        s.max_tier = src[i].max_tier;
        s.nchunks = tier_chunks(src[i].stride);
        s.chunk0 = t.count_stride;
        s.base_stride = tier_blocks(src[i].stride);
        s.blk_base = bases + (int64_t)batch * base_total;
        base_total += s.base_stride;
        t.count_stride += s.nchunks;
        max_chunks = max(max_chunks, s.nchunks);
    }
    t.nsrc = nsrc;
    t.tau_low = tau_low;
    t.tau_high = tau_high;
    t.h_cap = h.max_blocks * BT;
    t.m_cap = m.max_blocks * BT;
    t.counts = counts;
    t.n_high = n_high;
    t.n_mid = n_mid;
    const dim3 sgrid((unsigned)max_chunks, (unsigned)batch, (unsigned)nsrc);
    hipLaunchKernelGGL(tier_count_kernel, sgrid, dim3(256), 0, stream, t);
    hipLaunchKernelGGL(tier_write_kernel, sgrid, dim3(256), 0, stream, t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || max_blocks == 0) return e;
    MoveArgs a = {};
    for (int i = 0; i < nsrc; i++) {
        MoveSrc& s = a.src[i];
        s.f = src[i].f;
        s.pool = src[i].pool;
        s.bt = src[i].block_table;
        s.max_blocks = src[i].max_blocks;
        s.lens = src[i].view_lens;
        s.len_cap = t.src[i].len_cap;
        s.tiers = src[i].tiers;
        s.tier_stride = src[i].stride;
        s.blk_base = t.src[i].blk_base;
        s.base_stride = t.src[i].base_stride;
    }
    a.dst[0] = MoveDst{h.f, h.pool, h.block_table, h.max_blocks};
    a.dst[1] = MoveDst{m.f, m.pool, m.block_table, m.max_blocks};
    a.n_high = n_high;
    a.n_mid = n_mid;
    a.nsrc = nsrc;
    // V codes: 6-bit sources (HIGH copied, MID requantised) or 4-bit ones (MID copied)
    for (int i = 0; i < nsrc; i++)
        if (!(src[i].f.vb == 6 || (src[i].f.vb == 4 && m.f.vb == 4))) return hipErrorInvalidValue;
    if (h.f.vb != 6 || m.f.vb != 4) return hipErrorInvalidValue;
    // the destination segment (0 HIGH, 1 MID) that is source i itself, or -1
    int own[2] = {-1, -1};
    bool in_place = false;
    for (int i = 0; i < nsrc; i++) {
        if (h.pool == src[i].pool && h.block_table == src[i].block_table) own[i] = 0;
        if (m.pool == src[i].pool && m.block_table == src[i].block_table) own[i] = 1;
        in_place |= own[i] >= 0;
    }
    // runs per workgroup: as many as keep about 1024 workgroups in the grid
    // (fewer workgroup edges, whose words take atomics), at most CMP_S
    // (in place about 4096: its workgroups wait on earlier ones, and the
    // run count assumes every sequence at max_len)
    auto per_wg = [&](const TierSource* ss, int n, int64_t target) {
        int64_t runs = 0;
        for (int i = 0; i < n; i++) runs += (int64_t)batch * h.f.H * ((ss[i].max_len + BT * CMP_R - 1) / (BT * CMP_R));
        return (int32_t)std::max<int64_t>(1, std::min<int64_t>(CMP_S, runs / target));
    };
    auto go = [&](const MoveArgs& x, dim3 grid, bool ip) {
        auto run = [&](auto k) { hipLaunchKernelGGL(k, grid, dim3(256), 0, stream, x); };
        if (h.f.D == 64) {
            if (h.f.g == 64) ip ? run(tier_compact_ip_kernel<64, 64>) : run(tier_compact_kernel<64, 64, false>);
            else if (h.f.g == 32) ip ? run(tier_compact_ip_kernel<64, 32>) : run(tier_compact_kernel<64, 32, false>);
            else ip ? run(tier_compact_ip_kernel<64, 16>) : run(tier_compact16_kernel<64>);
        } else {
            if (h.f.g == 64) ip ? run(tier_compact_ip_kernel<128, 64>) : run(tier_compact_kernel<128, 64, false>);
            else if (h.f.g == 32) ip ? run(tier_compact_ip_kernel<128, 32>) : run(tier_compact_kernel<128, 32, false>);
            else ip ? run(tier_compact_ip_kernel<128, 16>) : run(tier_compact16_kernel<128>);
        }
    };
    if (!in_place) {
        a.per_wg = per_wg(src, nsrc, 1024);
        const int span = CMP_R * a.per_wg;
        go(a, dim3((unsigned)((max_blocks + span - 1) / span), (unsigned)h.f.H, (unsigned)(batch * nsrc)), false);
        return hipGetLastError();
    }
    // one source per launch, in destination order (MID first: the demoted
    // HIGH tokens land in MID blocks after the kept MID tokens); a source
    // compacted in place takes its workgroups' work from a ticket counter
    uint32_t* ticket = (uint32_t*)(bases + (int64_t)batch * base_total);
    uint32_t* flags = ticket + 2;
    for (int i = 0; i < nsrc; i++) {
        MoveArgs one = a;
        one.src[0] = a.src[i];
        one.nsrc = 1;
        one.per_wg = per_wg(&src[i], 1, own[i] < 0 ? 1024 : 4096);
        const int32_t nruns = max(1, (src[i].max_len + BT * CMP_R - 1) / (BT * CMP_R));
        const int32_t groups = (nruns + one.per_wg - 1) / one.per_wg;
        if (own[i] < 0) {
            go(one, dim3((unsigned)groups, (unsigned)h.f.H, (unsigned)batch), false);
        } else {
            if ((e = launch_fill_u32(ticket, 2 + (int64_t)batch * nruns, 0u, stream)) != hipSuccess) return e;
            one.ticket = ticket;
            one.flags = flags;
            one.flag_stride = nruns;
            one.inplace_seg = own[i];
            one.gx = groups;
            go(one, dim3((unsigned)((int64_t)groups * h.f.H * batch)), true);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace lkv
