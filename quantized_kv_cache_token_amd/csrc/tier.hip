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
//    writes their tiers and the source token of every destination position.
//    The first chunk writes the two counts (negative when a destination has
//    no room) and source 0's totals.
//  compact: one workgroup per (sequence, destination block, KV head,
//    destination).  It gathers its 64 destination rows: K rows, scales and
//    zeros copied bit for bit; V codes copied when the source holds the
//    destination's width, else (V6 -> V4) dequantised in fp32 and
//    requantised at 4 bits; then packs the channel-major V rows.
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
};

struct TierScanArgs {
    TierSrc src[2];  // in destination order
    int32_t nsrc;
    float tau_low, tau_high;
    int32_t h_cap, m_cap;
    int32_t* h_map;  // [batch][map_stride]: source token of each destination position
    int32_t* m_map;
    int32_t map_stride;
    int32_t* n_high;
    int32_t* n_mid;
    int2* counts;    // [batch][count_stride] (HIGH, MID): source 0's chunks, then source 1's
    int32_t count_stride;
    int2* bounds;    // [batch] (HIGH, MID) totals of source 0; null with one source
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
    const TierSrc& src = a.src[blockIdx.z];
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
    const TierSrc& src = a.src[z];
    if (c >= src.nchunks) return;
    const int len = max(0, min(src.lens[b], src.len_cap));
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // totals over every source, the counts that come before this chunk in
    // destination order (earlier sources, then earlier chunks), and the
    // totals of source 0
    const int self = src.chunk0 + c, n0 = a.src[0].nchunks;
    int th = 0, tm = 0, bh = 0, bm = 0, h0 = 0, m0 = 0;
    for (int i = lane; i < a.count_stride; i += 64) {
        const int2 v = a.counts[(int64_t)b * a.count_stride + i];
        th += v.x;
        tm += v.y;
        if (i < self) { bh += v.x; bm += v.y; }
        if (i < n0) { h0 += v.x; m0 += v.y; }
    }
    for (int o = 32; o > 0; o >>= 1) {
        th += __shfl_xor(th, o, 64);
        tm += __shfl_xor(tm, o, 64);
        bh += __shfl_xor(bh, o, 64);
        bm += __shfl_xor(bm, o, 64);
        h0 += __shfl_xor(h0, o, 64);
        m0 += __shfl_xor(m0, o, 64);
    }
    const bool fits = th <= a.h_cap && tm <= a.m_cap;
    if (z == 0 && c == 0 && tid == 0) {
        a.n_high[b] = fits ? th : -th;
        a.n_mid[b] = fits ? tm : -tm;
        if (a.bounds) a.bounds[b] = make_int2(h0, m0);
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
    int32_t* hs = a.h_map + (int64_t)b * a.map_stride;
    int32_t* ms = a.m_map + (int64_t)b * a.map_stride;
#pragma unroll
    for (int i = 0; i < TIER_PER; i++) {
        if (t[i] == 2) hs[ph++] = j0 + i;
        else if (t[i] == 1) ms[pm++] = j0 + i;
    }
}

struct CompactArgs {
    Fmt fs0, fs1;                 // source formats (the second only with two sources)
    const uint8_t* src_pool[2];
    const int32_t* src_bt[2];
    int32_t src_max_blocks[2];
    Fmt fh, fm;
    uint8_t* h_pool;
    const int32_t* h_bt;
    int32_t h_max_blocks;
    uint8_t* m_pool;
    const int32_t* m_bt;
    int32_t m_max_blocks;
    const int32_t* n_high;
    const int32_t* n_mid;
    const int32_t* h_map;
    const int32_t* m_map;
    int32_t map_stride;
    const int2* bounds;           // null with one source
    int32_t nblk;
};

constexpr int CU = 4;  // slots a wave keeps in flight

// One workgroup per (sequence, destination block, KV head, destination).
// Destination position p of a sequence comes from source 0 below that
// source's total for the destination (bounds), else from source 1.
template <int D>
__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a)
{
    constexpr int VPL = D / 64;
    const int seg = blockIdx.z;  // 0: HIGH -> h, 1: MID -> m
    const int b = blockIdx.x / a.nblk, lb = blockIdx.x % a.nblk, kvh = blockIdx.y;
    const int nh = a.n_high[b], nm = a.n_mid[b];
    if (nh < 0 || nm < 0) return;  // no room: nothing is written
    const int n = seg == 0 ? nh : nm;
    const int p0 = lb * BT;
    if (p0 >= n) return;
    const int cnt = min(BT, n - p0);
    const Fmt& fd = seg == 0 ? a.fh : a.fm;
    const int32_t* idx = (seg == 0 ? a.h_map : a.m_map) + (int64_t)b * a.map_stride + p0;
    const int32_t* dbt = seg == 0 ? a.h_bt : a.m_bt;
    const int32_t dmax = seg == 0 ? a.h_max_blocks : a.m_max_blocks;
    uint8_t* dpool = seg == 0 ? a.h_pool : a.m_pool;
    uint8_t* dch = dpool + ((int64_t)dbt[(int64_t)b * dmax + lb] * fd.H + kvh) * fd.chunk;
    const int bound = a.bounds ? (seg == 0 ? a.bounds[b].x : a.bounds[b].y) : 0x7FFFFFFF;

    // every slot's source, chunk and slot, resolved at once
    __shared__ const uint8_t* src_ch[BT];
    __shared__ int src_slot[BT];
    __shared__ int src_id[BT];
    if (threadIdx.x < cnt) {
        const int j = idx[threadIdx.x];
        const int sid = p0 + (int)threadIdx.x >= bound;
        const int64_t chunk = sid ? a.fs1.chunk : a.fs0.chunk;
        src_id[threadIdx.x] = sid;
        src_slot[threadIdx.x] = j % BT;
        src_ch[threadIdx.x] =
            a.src_pool[sid] + ((int64_t)a.src_bt[sid][(int64_t)b * a.src_max_blocks[sid] + j / BT] * fd.H + kvh) *
                                  chunk;
    }
    __syncthreads();

    __shared__ uint8_t vc[BT][D];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kw = fd.krow / 4;  // K words per row (<= 64), equal in every format here
    for (int s0 = wave; s0 < cnt; s0 += 4 * CU) {
        // loads of CU slots (s0, s0 + 4, ...; past the end: the last slot again)
        uint32_t kword[CU], vlo[CU][VPL], vhi[CU][VPL];
        float ks[CU], vs[CU][VPL];
        uint32_t kz[CU], vz[CU][VPL];
#pragma unroll
        for (int u = 0; u < CU; u++) {
            const int s = min(s0 + 4 * u, cnt - 1);
            const Fmt& fs = __builtin_amdgcn_readfirstlane(src_id[s]) ? a.fs1 : a.fs0;
            const uint8_t* sch = src_ch[s];
            const int sslot = src_slot[s];
            kword[u] = lane < kw ? ((const uint32_t*)(sch + fs.off_kc + sslot * fs.krow))[lane] : 0u;
            const int gl = min(lane, fs.ngroups - 1);
            ks[u] = ((const float*)(sch + fs.off_ks))[gl * BT + sslot];
            kz[u] = sch[fs.off_kz + gl * BT + sslot];
            const int bit = sslot * fs.vb;
#pragma unroll
            for (int i = 0; i < VPL; i++) {
                const int d = lane + 64 * i;
                const int gi = d / fs.g;
                // the two words that can hold the field (the second may be
                // the next row's first word, or the first metadata word:
                // still inside the chunk)
                const uint32_t* w = (const uint32_t*)(sch + fs.off_vc + d * fs.vrow) + (bit >> 5);
                vlo[u][i] = w[0];
                vhi[u][i] = w[1];
                vs[u][i] = ((const float*)(sch + fs.off_vs))[gi * BT + sslot];
                vz[u][i] = sch[fs.off_vz + gi * BT + sslot];
            }
        }
#pragma unroll
        for (int u = 0; u < CU; u++) {
            const int s = s0 + 4 * u;
            if (s >= cnt) break;
            const Fmt& fs = __builtin_amdgcn_readfirstlane(src_id[s]) ? a.fs1 : a.fs0;
            const int sslot = src_slot[s];
            // K row, K scales, K zeros: bit for bit
            if (lane < kw) ((uint32_t*)(dch + fd.off_kc + s * fd.krow))[lane] = kword[u];
            if (lane < fs.ngroups) {
                ((float*)(dch + fd.off_ks))[lane * BT + s] = ks[u];
                dch[fd.off_kz + lane * BT + s] = (uint8_t)kz[u];
            }
            const int sh = (sslot * fs.vb) & 31;
            const bool same = fs.vb == fd.vb;
#pragma unroll
            for (int i = 0; i < VPL; i++) {
                const int d = lane + 64 * i;
                const int gi = d / fs.g;
                const uint64_t x64 = ((uint64_t)vhi[u][i] << 32) | vlo[u][i];
                const uint32_t code = (uint32_t)(x64 >> sh) & ((1u << fs.vb) - 1u);
                if (same) {  // V codes, scale and zero copied
                    vc[s][d] = (uint8_t)code;
                    if ((d % fs.g) == 0) {
                        ((float*)(dch + fd.off_vs))[gi * BT + s] = vs[u][i];
                        dch[fd.off_vz + gi * BT + s] = (uint8_t)vz[u][i];
                    }
                } else {  // 6 -> 4 bits: dequantised, one fp32 rounding, requantised
                    const float x = (float)((int)code - (int)vz[u][i]) * vs[u][i];
                    float s4;
                    int z4;
                    const int c4 = quantize_lane(x, fd.g, fd.vb, &s4, &z4);
                    vc[s][d] = (uint8_t)c4;
                    if ((d % fd.g) == 0) {
                        ((float*)(dch + fd.off_vs))[gi * BT + s] = s4;
                        dch[fd.off_vz + gi * BT + s] = (uint8_t)z4;
                    }
                }
            }
        }
    }
    __syncthreads();
    const int wv = BT * fd.vb / 32;
    for (int i = threadIdx.x; i < D * wv; i += blockDim.x) {
        const int d = i / wv, w = i % wv;
        const uint32_t word = pack_word(w, fd.vb, 0, cnt, [&](int s) { return (uint32_t)vc[s][d]; });
        ((uint32_t*)(dch + fd.off_vc + d * fd.vrow))[w] = word;
    }
}

hipError_t launch_tiering(const TierSource* src, int nsrc, float tau_low, float tau_high, const TierDest& h,
                          const TierDest& m, int32_t* n_high, int32_t* n_mid, int32_t batch, void* workspace,
                          hipStream_t stream)
{
    if (batch == 0) return hipSuccess;
    TierScanArgs t = {};
    int32_t max_chunks = 0, map_stride = 0, max_len = 0;
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
        t.count_stride += s.nchunks;
        max_chunks = max(max_chunks, s.nchunks);
        map_stride += src[i].stride;
        max_len += src[i].max_len;
    }
    t.nsrc = nsrc;
    t.tau_low = tau_low;
    t.tau_high = tau_high;
    t.h_cap = h.max_blocks * BT;
    t.m_cap = m.max_blocks * BT;
    t.map_stride = map_stride;
    t.h_map = (int32_t*)workspace;
    t.m_map = t.h_map + (int64_t)batch * map_stride;
    t.counts = (int2*)(t.m_map + (int64_t)batch * map_stride);
    t.bounds = nsrc == 2 ? t.counts + (int64_t)batch * t.count_stride : nullptr;
    t.n_high = n_high;
    t.n_mid = n_mid;
    const dim3 sgrid((unsigned)max_chunks, (unsigned)batch, (unsigned)nsrc);
    hipLaunchKernelGGL(tier_count_kernel, sgrid, dim3(256), 0, stream, t);
    hipLaunchKernelGGL(tier_write_kernel, sgrid, dim3(256), 0, stream, t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || max_len == 0) return e;
    CompactArgs a = {};
    a.fs0 = src[0].f;
    a.fs1 = nsrc == 2 ? src[1].f : src[0].f;
    for (int i = 0; i < nsrc; i++) {
        a.src_pool[i] = src[i].pool;
        a.src_bt[i] = src[i].block_table;
        a.src_max_blocks[i] = src[i].max_blocks;
    }
    a.fh = h.f;
    a.fm = m.f;
    a.h_pool = h.pool;
    a.h_bt = h.block_table;
    a.h_max_blocks = h.max_blocks;
    a.m_pool = m.pool;
    a.m_bt = m.block_table;
    a.m_max_blocks = m.max_blocks;
    a.n_high = n_high;
    a.n_mid = n_mid;
    a.h_map = t.h_map;
    a.m_map = t.m_map;
    a.map_stride = map_stride;
    a.bounds = t.bounds;
    // destination blocks that can hold a survivor
    a.nblk = min((max_len + BT - 1) / BT, max(h.max_blocks, m.max_blocks));
    dim3 grid((unsigned)(batch * a.nblk), (unsigned)h.f.H, 2);
    if (h.f.D == 64) hipLaunchKernelGGL(compact_kernel<64>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(compact_kernel<128>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lkv
