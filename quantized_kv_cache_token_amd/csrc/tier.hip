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
//  tier_move: one workgroup per (8 consecutive source chunks, KV head,
//    sequence, source).  Each source chunk is read once, whole and
//    coalesced; its survivors go to consecutive destination positions.  K
//    rows, scales and zeros are stored straight from the loaded pieces; V
//    codes are copied (same width) or dequantised in fp32 and requantised
//    at 4 bits (V6 -> V4) into an LDS block of destination codes, which is
//    packed into the channel-major rows when it fills or the workgroup ends.
//    Only the words a neighbouring workgroup also writes are merged with
//    atomics.
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

constexpr int MOVE_CHUNKS = 8;   // source chunks per workgroup, in token order
constexpr int MOVE_PIECES = 5;   // 16-byte pieces per thread of one chunk (chunks up to 20 KiB)
constexpr int MOVE_META = 5120;  // bytes of the scale and zero sections (D / g = 8 groups)

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
};

__device__ __forceinline__ uint8_t* dst_chunk(const MoveDst& d, int b, int pos, int kvh)
{
    return d.pool + ((int64_t)d.bt[(int64_t)b * d.max_blocks + pos / BT] * d.f.H + kvh) * d.f.chunk;
}

// Packs destination slots [slo, shi) of every channel row from the staged
// codes into chunk dch; words shared with slots outside the range are
// merged with atomics.
template <int D>
__device__ __forceinline__ void flush_block(const Fmt& fd, uint8_t* dch, const uint8_t (*st)[VPITCH], int slo, int shi)
{
    if (fd.vb == 6) pack_v_rows<6, 16, 3, D>(st, dch, fd.off_vc, fd.vrow, slo, shi);
    else pack_v_rows<4, 8, 1, D>(st, dch, fd.off_vc, fd.vrow, slo, shi);
}

// Where slot s of a source chunk goes: its segment (0 HIGH, 1 MID, -1
// evicted), destination chunk and slot.  The survivors of segment i (mask
// mk_i) take consecutive positions from pos_i in slot order; a chunk's
// survivors span at most two destination blocks (dA_i: pos_i's block, dB_i:
// the next one).
__device__ __forceinline__ int slot_dest(int s, uint64_t mk0, uint64_t mk1, int pos0, int pos1, uint8_t* dA0,
                                         uint8_t* dB0, uint8_t* dA1, uint8_t* dB1, uint8_t** dch, int* ds)
{
    const uint64_t bit = 1ull << s, lt = bit - 1ull;
    if (mk0 & bit) {
        const int P = pos0 + __popcll(mk0 & lt);
        *dch = P / BT == pos0 / BT ? dA0 : dB0;
        *ds = P % BT;
        return 0;
    }
    if (mk1 & bit) {
        const int P = pos1 + __popcll(mk1 & lt);
        *dch = P / BT == pos1 / BT ? dA1 : dB1;
        *ds = P % BT;
        return 1;
    }
    return -1;
}

// V codes of survivor ranks [r0, r1) of one segment, copied at the source
// width into staged slots r + sh of the channel-major stage.
template <int D>
__device__ __forceinline__ void copy_codes(uint8_t (*st)[VPITCH], const uint8_t* src_of, const uint32_t* vsrc,
                                           int vrow_w, int vb, int r0, int r1, int sh)
{
    const int cnt = (r1 - r0) * D;
    for (int i = threadIdx.x; i < cnt; i += 256) {
        const int r = r0 + i / D, d = i % D;
        st[d][r + sh] = (uint8_t)get_field(vsrc + d * vrow_w, src_of[r], vb);
    }
}

// MID survivor ranks [r0, r1) from 6-bit V: dequantised in fp32 and
// requantised at the destination width, four tokens per wave at a time
// (lane: channels P * lane + p); codes into staged slots r + sh, scales and
// zeros straight to the destination.
template <int D, int GS>
__device__ __forceinline__ void requant_codes_g(uint8_t (*st)[VPITCH], const uint8_t* src_of, const uint32_t* vsrc,
                                              int vrow_w, const Fmt& fs, const Fmt& fm, const float* m_vs,
                                              const uint8_t* m_vz, int pos, uint8_t* dA, uint8_t* dB, int r0, int r1,
                                              int sh)
{
    constexpr int P = D / 64, T = 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int rb = r0 + T * wave; rb < r1; rb += 4 * T) {
        float x[T][P];
        QRow<P> q[T];
#pragma unroll
        for (int t = 0; t < T; t++) {
            const int s = src_of[min(rb + t, r1 - 1)];
#pragma unroll
            for (int p = 0; p < P; p++) {
                const int d = P * lane + p, gi = d / fs.g;
                const uint32_t code = get_field(vsrc + d * vrow_w, s, fs.vb);
                x[t][p] = (float)((int)code - (int)m_vz[gi * BT + s]) * m_vs[gi * BT + s];  // one fp32 rounding
            }
        }
#pragma unroll
        for (int t = 0; t < T; t++) quantize_fast<P, GS>(x[t], fm.vb, q[t]);
#pragma unroll
        for (int t = 0; t < T; t++)
            if (q[t].slow) quantize_exact<P>(x[t], fm.vb, q[t]);
#pragma unroll
        for (int t = 0; t < T; t++) {
            const int r = rb + t;
            if (r >= r1) break;
            const int P_ = pos + r;
            uint8_t* dch = P_ / BT == pos / BT ? dA : dB;
#pragma unroll
            for (int p = 0; p < P; p++) st[P * lane + p][r + sh] = (uint8_t)q[t].q[p];
            if ((P * lane) % GS == 0) {
                const int gi = P * lane / GS;
                ((float*)(dch + fm.off_vs))[gi * BT + P_ % BT] = q[t].s;
                dch[fm.off_vz + gi * BT + P_ % BT] = (uint8_t)q[t].z;
            }
        }
    }
}

template <int D>
__device__ __forceinline__ void requant_codes(uint8_t (*st)[VPITCH], const uint8_t* src_of, const uint32_t* vsrc,
                                              int vrow_w, const Fmt& fs, const Fmt& fm, const float* m_vs,
                                              const uint8_t* m_vz, int pos, uint8_t* dA, uint8_t* dB, int r0, int r1,
                                              int sh)
{
    if (fm.g == 64) requant_codes_g<D, 64>(st, src_of, vsrc, vrow_w, fs, fm, m_vs, m_vz, pos, dA, dB, r0, r1, sh);
    else if (fm.g == 32) requant_codes_g<D, 32>(st, src_of, vsrc, vrow_w, fs, fm, m_vs, m_vz, pos, dA, dB, r0, r1, sh);
    else requant_codes_g<D, 16>(st, src_of, vsrc, vrow_w, fs, fm, m_vs, m_vz, pos, dA, dB, r0, r1, sh);
}

template <int D>
__global__ __launch_bounds__(256) void tier_move_kernel(MoveArgs a)
{
    __shared__ uint32_t vsrc[D * 12 + 4];        // the V section (up to 6-bit), plus slack for straddling reads
    __shared__ uint32_t meta[MOVE_META / 4];     // K scales, V scales, K zeros, V zeros
    __shared__ uint8_t stage[2][D][VPITCH];      // destination codes of the current HIGH / MID block
    __shared__ uint8_t src_of[4][2][BT];         // per wave: source slot of each survivor rank

    const int si = blockIdx.z % a.nsrc, b = blockIdx.z / a.nsrc, kvh = blockIdx.y;
    if (a.n_high[b] < 0 || a.n_mid[b] < 0) return;  // no room: nothing is written
    const MoveSrc& S = si == 0 ? a.src[0] : a.src[1];
    const Fmt& fs = S.f;
    const int len = max(0, min(S.lens[b], S.len_cap));
    const int nblocks = (len + BT - 1) / BT;
    const int c0 = blockIdx.x * MOVE_CHUNKS;
    if (c0 >= nblocks) return;
    const int c1 = min(nblocks, c0 + MOVE_CHUNKS);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int2 base = S.blk_base[(int64_t)b * S.base_stride + c0];
    // next destination position of each segment, and the first position this
    // workgroup staged in the segment's current block
    int pos0 = base.x, pos1 = base.y, lo0 = base.x, lo1 = base.y;
    const int krows = BT * fs.krow, vbytes = D * fs.vrow;
    const int npieces = (int)(fs.chunk / 16);
    const int vrow_w = fs.vrow / 4;
    const float* m_ks = (const float*)meta;
    const float* m_vs = (const float*)((const uint8_t*)meta + (fs.off_vs - fs.off_ks));
    const uint8_t* m_kz = (const uint8_t*)meta + (fs.off_kz - fs.off_ks);
    const uint8_t* m_vz = (const uint8_t*)meta + (fs.off_vz - fs.off_ks);
    // destination layouts: both hold the source's K format, so K rows sit at
    // the same offsets; the scale and zero sections differ with the V width
    const Fmt& fh = a.dst[0].f;
    const Fmt& fm = a.dst[1].f;
    const bool copy_m = fm.vb == fs.vb;  // MID survivors keep their V codes (a MID source)

    // a chunk's tiers and its pieces are requested together (the tiers and
    // block of the next chunk one iteration ahead)
    auto tiers_of = [&](int c) __attribute__((always_inline)) {
        return lane < min(BT, len - c * BT) ? (int)S.tiers[(int64_t)b * S.tier_stride + c * BT + lane] : 0;
    };
    int t_next = tiers_of(c0);
    int blk_next = S.bt[(int64_t)b * S.max_blocks + c0];
    for (int c = c0; c < c1; c++) {
        const uint8_t* sch = S.pool + ((int64_t)blk_next * fs.H + kvh) * fs.chunk;
        uint4 pc[MOVE_PIECES];
#pragma unroll
        for (int k = 0; k < MOVE_PIECES; k++) {
            const int p = tid + 256 * k;
            pc[k] = p < npieces ? ((const uint4*)sch)[p] : make_uint4(0u, 0u, 0u, 0u);
        }
        // tiers of the chunk's 64 slots; every wave derives the same masks
        const int t = t_next;
        if (c + 1 < c1) {
            t_next = tiers_of(c + 1);
            blk_next = S.bt[(int64_t)b * S.max_blocks + c + 1];
        }
        const uint64_t mk0 = __ballot(t == 2), mk1 = __ballot(t == 1);
        const uint64_t below = (1ull << lane) - 1ull;
        if (t == 2) src_of[wave][0][__popcll(mk0 & below)] = (uint8_t)lane;
        else if (t == 1) src_of[wave][1][__popcll(mk1 & below)] = (uint8_t)lane;
        const int n0 = __popcll(mk0), n1 = __popcll(mk1);
        if (n0 + n1 == 0) continue;
        // destination chunks: the block of each segment's next position and
        // the one after it
        uint8_t *dA0 = nullptr, *dB0 = nullptr, *dA1 = nullptr, *dB1 = nullptr;
        if (n0) {
            dA0 = dst_chunk(a.dst[0], b, pos0, kvh);
            dB0 = pos0 % BT + n0 > BT ? dst_chunk(a.dst[0], b, pos0 + BT, kvh) : dA0;
        }
        if (n1) {
            dA1 = dst_chunk(a.dst[1], b, pos1, kvh);
            dB1 = pos1 % BT + n1 > BT ? dst_chunk(a.dst[1], b, pos1 + BT, kvh) : dA1;
        }
        __syncthreads();  // the previous chunk's readers of vsrc and meta are done
#pragma unroll
        for (int k = 0; k < MOVE_PIECES; k++) {
            const int off = 16 * (tid + 256 * k);
            if (off >= 16 * npieces) continue;
            if (off >= fs.off_ks) {
                *(uint4*)((uint8_t*)meta + (off - fs.off_ks)) = pc[k];
            } else if (off >= fs.off_vc) {
                if (off < fs.off_vc + vbytes) *(uint4*)((uint8_t*)vsrc + (off - fs.off_vc)) = pc[k];
            } else if (off < krows) {  // a K row piece: stored straight to its survivor's row
                uint8_t* dch;
                int ds;
                if (slot_dest(off / fs.krow, mk0, mk1, pos0, pos1, dA0, dB0, dA1, dB1, &dch, &ds) >= 0)
                    *(uint4*)(dch + fh.off_kc + ds * fh.krow + off % fs.krow) = pc[k];
            }
        }
        __syncthreads();
        // K scales and zeros of every survivor; V scales and zeros where V is copied
        for (int i = tid; i < fs.ngroups * BT; i += 256) {
            uint8_t* dch;
            int ds;
            const int seg = slot_dest(i % BT, mk0, mk1, pos0, pos1, dA0, dB0, dA1, dB1, &dch, &ds);
            if (seg < 0) continue;
            ds += i / BT * BT;
            ((float*)(dch + (seg == 0 ? fh.off_ks : fm.off_ks)))[ds] = m_ks[i];
            dch[(seg == 0 ? fh.off_kz : fm.off_kz) + ds] = m_kz[i];
            if (seg == 0 || copy_m) {
                ((float*)(dch + (seg == 0 ? fh.off_vs : fm.off_vs)))[ds] = m_vs[i];
                dch[(seg == 0 ? fh.off_vz : fm.off_vz) + ds] = m_vz[i];
            }
        }
        // V codes of each segment into its staged block; a block that fills
        // is packed out and the rest of the chunk's survivors start the next
        // one.  HIGH codes are always copied (6-bit to 6-bit).
        if (n0) {
            const int first = min(n0, BT - pos0 % BT);
            copy_codes<D>(stage[0], src_of[wave][0], vsrc, vrow_w, fs.vb, 0, first, pos0 % BT);
            if (pos0 % BT + n0 >= BT) {  // the block is complete
                __syncthreads();
                flush_block<D>(fh, dA0, stage[0], lo0 - pos0 / BT * BT, BT);
                __syncthreads();
                lo0 = (pos0 / BT + 1) * BT;
                if (first < n0) copy_codes<D>(stage[0], src_of[wave][0], vsrc, vrow_w, fs.vb, first, n0, -first);
            }
            pos0 += n0;
        }
        if (n1) {
            const int first = min(n1, BT - pos1 % BT);
            if (copy_m)
                copy_codes<D>(stage[1], src_of[wave][1], vsrc, vrow_w, fs.vb, 0, first, pos1 % BT);
            else
                requant_codes<D>(stage[1], src_of[wave][1], vsrc, vrow_w, fs, fm, m_vs, m_vz, pos1, dA1, dB1,
                                 0, first, pos1 % BT);
            if (pos1 % BT + n1 >= BT) {
                __syncthreads();
                flush_block<D>(fm, dA1, stage[1], lo1 - pos1 / BT * BT, BT);
                __syncthreads();
                lo1 = (pos1 / BT + 1) * BT;
                if (first < n1) {
                    if (copy_m)
                        copy_codes<D>(stage[1], src_of[wave][1], vsrc, vrow_w, fs.vb, first, n1, -first);
                    else
                        requant_codes<D>(stage[1], src_of[wave][1], vsrc, vrow_w, fs, fm, m_vs, m_vz, pos1, dA1,
                                         dB1, first, n1, -first);
                }
            }
            pos1 += n1;
        }
    }
    // the partly filled last block of each segment
    if (pos0 > lo0) {
        __syncthreads();
        const int blk0 = lo0 / BT * BT;
        flush_block<D>(fh, dst_chunk(a.dst[0], b, lo0, kvh), stage[0], lo0 - blk0, pos0 - blk0);
    }
    if (pos1 > lo1) {
        __syncthreads();
        const int blk0 = lo1 / BT * BT;
        flush_block<D>(fm, dst_chunk(a.dst[1], b, lo1, kvh), stage[1], lo1 - blk0, pos1 - blk0);
    }
}

hipError_t launch_tiering(const TierSource* src, int nsrc, float tau_low, float tau_high, const TierDest& h,
                          const TierDest& m, int32_t* n_high, int32_t* n_mid, int32_t batch, void* workspace,
                          hipStream_t stream)
{
    if (batch == 0) return hipSuccess;
    for (int i = 0; i < nsrc; i++)  // every quantised format fits the move kernel's staging
        if (src[i].f.chunk > 16 * 256 * MOVE_PIECES || src[i].f.chunk - src[i].f.off_ks > MOVE_META ||
            src[i].f.vb > 6 || src[i].f.D != h.f.D)
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
        s.len_cap = min(src[i].stride, src[i].max_blocks * BT);
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
    const dim3 grid((unsigned)((max_blocks + MOVE_CHUNKS - 1) / MOVE_CHUNKS), (unsigned)h.f.H,
                    (unsigned)(batch * nsrc));
    if (h.f.D == 64) hipLaunchKernelGGL(tier_move_kernel<64>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(tier_move_kernel<128>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lkv
