// tier.hip -- attention-aware tier update (Super KV Compression page, second
// layer), built with -ffp-contract=off.
//
//  classify_scan: one workgroup per sequence.  Tier of each token from its
//    score (HIGH >= tau_high, MID >= tau_low, LOW otherwise), block-wide
//    exclusive scans of the HIGH and MID flags (stable order), the source
//    token index of every destination position, and the two counts.
//  compact: one workgroup per (sequence, destination block, KV head,
//    segment).  It gathers its 64 destination rows: K rows, scales and zeros
//    copied bit for bit; V6 codes copied (HIGH) or dequantised in fp32 and
//    requantised at 4 bits (MID); then packs the channel-major V rows.
#include <hip/hip_fp16.h>

#include "lkv_internal.h"
#include "quant_device.h"

namespace lkv {

__global__ __launch_bounds__(1024) void classify_scan_kernel(
    const float* __restrict__ scores, int32_t stride, int32_t len_cap, const int32_t* __restrict__ lens,
    float tau_low, float tau_high, int32_t h_cap, int32_t m_cap, uint8_t* __restrict__ tiers,
    int32_t* __restrict__ h_src, int32_t* __restrict__ m_src, int32_t* __restrict__ n_high,
    int32_t* __restrict__ n_mid)
{
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int len = max(0, min(lens[b], len_cap));  // out-of-contract lengths are clamped
    const int per = (len + 1023) / 1024;
    const int j0 = min(tid * per, len), j1 = min(j0 + per, len);
    const float* sc = scores + (int64_t)b * stride;
    int ch = 0, cm = 0;
    for (int j = j0; j < j1; j++) {
        const float s = sc[j];
        ch += s >= tau_high;
        cm += (s >= tau_low) & (s < tau_high);
    }
    // exclusive scan of (ch, cm) over the 1024 threads
    __shared__ int wsum_h[16], wsum_m[16];
    const int lane = tid & 63, wave = tid >> 6;
    int ih = ch, im = cm;
    for (int o = 1; o < 64; o <<= 1) {
        const int th = __shfl_up(ih, o, 64), tm = __shfl_up(im, o, 64);
        if (lane >= o) { ih += th; im += tm; }
    }
    if (lane == 63) { wsum_h[wave] = ih; wsum_m[wave] = im; }
    __syncthreads();
    int base_h = 0, base_m = 0, tot_h = 0, tot_m = 0;
    for (int w = 0; w < 16; w++) {
        if (w < wave) { base_h += wsum_h[w]; base_m += wsum_m[w]; }
        tot_h += wsum_h[w];
        tot_m += wsum_m[w];
    }
    int ph = base_h + ih - ch, pm = base_m + im - cm;
    const bool fits = tot_h <= h_cap && tot_m <= m_cap;
    uint8_t* t = tiers + (int64_t)b * stride;
    for (int j = j0; j < j1; j++) {
        const float s = sc[j];
        const int tier = s >= tau_high ? 2 : (s >= tau_low ? 1 : 0);
        t[j] = (uint8_t)tier;
        if (!fits) continue;
        if (tier == 2) h_src[(int64_t)b * stride + ph++] = j;
        else if (tier == 1) m_src[(int64_t)b * stride + pm++] = j;
    }
    if (tid == 0) {
        n_high[b] = fits ? tot_h : -tot_h;
        n_mid[b] = fits ? tot_m : -tot_m;
    }
}

struct CompactArgs {
    Fmt fs, fh, fm;
    const uint8_t* src_pool;
    const int32_t* src_bt;
    int32_t src_max_blocks;
    uint8_t* h_pool;
    const int32_t* h_bt;
    int32_t h_max_blocks;
    uint8_t* m_pool;
    const int32_t* m_bt;
    int32_t m_max_blocks;
    const int32_t* n_high;
    const int32_t* n_mid;
    const int32_t* h_src;
    const int32_t* m_src;
    int32_t stride;
    int32_t nblk;
};

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
    const Fmt& fs = a.fs;
    const Fmt& fd = seg == 0 ? a.fh : a.fm;
    const int32_t* idx = (seg == 0 ? a.h_src : a.m_src) + (int64_t)b * a.stride + p0;
    const int32_t* dbt = seg == 0 ? a.h_bt : a.m_bt;
    const int32_t dmax = seg == 0 ? a.h_max_blocks : a.m_max_blocks;
    uint8_t* dpool = seg == 0 ? a.h_pool : a.m_pool;
    uint8_t* dch = dpool + ((int64_t)dbt[(int64_t)b * dmax + lb] * fd.H + kvh) * fd.chunk;

    __shared__ uint8_t vc[BT][D];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int s = wave; s < cnt; s += 4) {
        const int j = idx[s];
        const int sslot = j % BT;
        const uint8_t* sch =
            a.src_pool + ((int64_t)a.src_bt[(int64_t)b * a.src_max_blocks + j / BT] * fs.H + kvh) * fs.chunk;
        // K row, K scales, K zeros: bit for bit
        const uint32_t* krow_s = (const uint32_t*)(sch + fs.off_kc + sslot * fs.krow);
        uint32_t* krow_d = (uint32_t*)(dch + fd.off_kc + s * fd.krow);
        for (int w = lane; w < fs.krow / 4; w += 64) krow_d[w] = krow_s[w];
        if (lane < fs.ngroups) {
            ((float*)(dch + fd.off_ks))[lane * BT + s] = ((const float*)(sch + fs.off_ks))[lane * BT + sslot];
            dch[fd.off_kz + lane * BT + s] = sch[fs.off_kz + lane * BT + sslot];
        }
        if (seg == 0) {
#pragma unroll
            for (int i = 0; i < VPL; i++) {
                const int d = lane + 64 * i;
                vc[s][d] = (uint8_t)get_field((const uint32_t*)(sch + fs.off_vc + d * fs.vrow), sslot, fs.vb);
            }
            if (lane < fs.ngroups) {
                ((float*)(dch + fd.off_vs))[lane * BT + s] = ((const float*)(sch + fs.off_vs))[lane * BT + sslot];
                dch[fd.off_vz + lane * BT + s] = sch[fs.off_vz + lane * BT + sslot];
            }
        } else {
#pragma unroll
            for (int i = 0; i < VPL; i++) {
                const int d = lane + 64 * i;
                const int gi = d / fs.g;
                const uint32_t c6 = get_field((const uint32_t*)(sch + fs.off_vc + d * fs.vrow), sslot, fs.vb);
                const float s6 = ((const float*)(sch + fs.off_vs))[gi * BT + sslot];
                const int z6 = sch[fs.off_vz + gi * BT + sslot];
                const float x = (float)((int)c6 - z6) * s6;  // one fp32 rounding
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
    __syncthreads();
    const int wv = BT * fd.vb / 32;
    for (int i = threadIdx.x; i < D * wv; i += blockDim.x) {
        const int d = i / wv, w = i % wv;
        const uint32_t word = pack_word(w, fd.vb, 0, cnt, [&](int s) { return (uint32_t)vc[s][d]; });
        ((uint32_t*)(dch + fd.off_vc + d * fd.vrow))[w] = word;
    }
}

hipError_t launch_tier_update(const Fmt& fs, const uint8_t* src_pool, const int32_t* src_bt,
                              const int32_t* src_lens, int32_t src_max_blocks, int32_t max_len,
                              const float* scores, int32_t stride, float tau_low, float tau_high,
                              const Fmt& fh, uint8_t* h_pool, const int32_t* h_bt, int32_t h_max_blocks,
                              const Fmt& fm, uint8_t* m_pool, const int32_t* m_bt, int32_t m_max_blocks,
                              int32_t* n_high, int32_t* n_mid, uint8_t* tiers, int32_t batch,
                              int32_t* h_src, int32_t* m_src, hipStream_t stream)
{
    if (batch == 0) return hipSuccess;
    hipLaunchKernelGGL(classify_scan_kernel, dim3((unsigned)batch), dim3(1024), 0, stream, scores, stride,
                       min(stride, src_max_blocks * BT), src_lens, tau_low, tau_high, h_max_blocks * BT, m_max_blocks * BT, tiers, h_src, m_src,
                       n_high, n_mid);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || max_len == 0) return e;
    CompactArgs a;
    a.fs = fs;
    a.fh = fh;
    a.fm = fm;
    a.src_pool = src_pool;
    a.src_bt = src_bt;
    a.src_max_blocks = src_max_blocks;
    a.h_pool = h_pool;
    a.h_bt = h_bt;
    a.h_max_blocks = h_max_blocks;
    a.m_pool = m_pool;
    a.m_bt = m_bt;
    a.m_max_blocks = m_max_blocks;
    a.n_high = n_high;
    a.n_mid = n_mid;
    a.h_src = h_src;
    a.m_src = m_src;
    a.stride = stride;
    a.nblk = (max_len + BT - 1) / BT;
    dim3 grid((unsigned)(batch * a.nblk), (unsigned)fs.H, 2);
    if (fs.D == 64) hipLaunchKernelGGL(compact_kernel<64>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(compact_kernel<128>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lkv
