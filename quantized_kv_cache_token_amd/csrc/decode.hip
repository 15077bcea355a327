// decode.hip -- split-K decode attention over the packed cache (generic
// vector-ALU kernel, every format and query dtype) and the merge of split
// partials.
//
// Work unit: one wave per (split, KV head, sequence).  A split walks its
// 64-token blocks in order; lane j holds token j of the block for the scores,
// and channels lane + 64 i for the V accumulation.  Per block and query head
// the running maximum m and sum L are updated (online softmax), the sparse-V
// rule of the Super KV Compression page (third layer) drops the V term of a
// token whose exp(s - m) < tau_low * L, and the accumulators are rescaled.
// The partial (o[D], m, L) of every split is written to the workspace; the
// combine kernel merges them.
#include <hip/hip_fp16.h>

#include <algorithm>

#include "lkv_internal.h"
#include "merge128.h"
#include "quant_device.h"

namespace lkv {

struct SplitArgs {
    SegArgs seg;
    const void* q;
    int32_t q_dtype;
    int32_t num_q_heads;
    int32_t split_tokens;
    int32_t total_splits;
    float score_scale;  // sm_scale * log2(e): scores are kept in base 2
    float tau_low;
    float* partials;
};

__device__ __forceinline__ float wave_max(float x)
{
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x)
{
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// Dequantised K element (token slot j, channel d) and V element.
__device__ __forceinline__ float deq_k(const uint8_t* ch, const Fmt& f, int j, int d)
{
    const uint32_t c = get_field((const uint32_t*)(ch + f.off_kc + j * f.krow), d, f.kb);
    if (f.fp16) return __half2float(__ushort_as_half((uint16_t)c));
    const int gi = d / f.g;
    const float s = ((const float*)(ch + f.off_ks))[gi * BT + j];
    const int z = ch[f.off_kz + gi * BT + j];
    return (float)((int)c - z) * s;
}
__device__ __forceinline__ float deq_v(const uint8_t* ch, const Fmt& f, int j, int d)
{
    const uint32_t c = get_field((const uint32_t*)(ch + f.off_vc + d * f.vrow), j, f.vb);
    if (f.fp16) return __half2float(__ushort_as_half((uint16_t)c));
    const int gi = d / f.g;
    const float s = ((const float*)(ch + f.off_vs))[gi * BT + j];
    const int z = ch[f.off_vz + gi * BT + j];
    return (float)((int)c - z) * s;
}

template <int D, int G>
__global__ __launch_bounds__(64) void split_valu_kernel(SplitArgs a)
{
    constexpr int VPL = D / 64;
    const SegArgs& sg = a.seg;
    const Fmt& f = sg.f;
    const int sp = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int len = max(0, min(entry_len(sg, b), sg.len_cap));  // out-of-contract lengths are clamped
    const int t0 = sp * a.split_tokens;
    const int t1 = min(t0 + a.split_tokens, len);
    if (t1 <= t0) {  // a split past the end: only (m, L) = (-inf, 0), its o row is never read
        if (lane < G) {
            float* p = a.partials +
                       (((int64_t)b * a.num_q_heads + kvh * G + lane) * a.total_splits + sg.split_base + sp) * (D + 2);
            p[D] = -INFINITY;
            p[D + 1] = 0.0f;
        }
        return;
    }

    __shared__ float qs[G][D];
    __shared__ float ps[G][BT];
    for (int i = lane; i < G * D; i += 64) {
        const int h = i / D, d = i % D;
        qs[h][d] = load_as_float(a.q, ((int64_t)b * a.num_q_heads + kvh * G + h) * D + d, a.q_dtype);
    }
    __syncthreads();

    float m[G], L[G], o[G][VPL];
#pragma unroll
    for (int h = 0; h < G; h++) {
        m[h] = -INFINITY;
        L[h] = 0.0f;
#pragma unroll
        for (int i = 0; i < VPL; i++) o[h][i] = 0.0f;
    }

    for (int bs = t0; bs < t1; bs += BT) {
        const int64_t blk = sg.block_table[(int64_t)entry_seq(sg, b) * sg.max_blocks + bs / BT];
        const uint8_t* ch = sg.pool + (blk * f.H + kvh) * f.chunk;
        const int nlive = min(BT, t1 - bs);
        const bool live = lane < nlive;
        float s[G];
#pragma unroll
        for (int h = 0; h < G; h++) s[h] = 0.0f;
        if (live) {
            for (int d = 0; d < D; d++) {
                const float kh = deq_k(ch, f, lane, d);
#pragma unroll
                for (int h = 0; h < G; h++) s[h] += qs[h][d] * kh;
            }
            if (f.k_norm) {  // direction-preserving K: the key is r * k_hat
                const float r = ((const float*)(ch + f.off_kn))[lane];
#pragma unroll
                for (int h = 0; h < G; h++) s[h] *= r;
            }
        }
#pragma unroll
        for (int h = 0; h < G; h++) {
            const float sc = live ? s[h] * a.score_scale : -INFINITY;
            if (sg.scores != nullptr && live)
                sg.scores[((int64_t)b * a.num_q_heads + kvh * G + h) * sg.score_stride + sg.tok_base + bs + lane] = sc;
            const float m_new = fmaxf(m[h], wave_max(sc));
            const float e = live ? exp2f(sc - m_new) : 0.0f;
            const float alpha = exp2f(m[h] - m_new);
            L[h] = L[h] * alpha + wave_sum(e);
            m[h] = m_new;
            const bool skip = a.tau_low > 0.0f && e < a.tau_low * L[h];
            ps[h][lane] = skip ? 0.0f : e;
            if (sg.skip_mask != nullptr && skip && live)
                mark_skipped(sg.skip_mask + ((int64_t)b * a.num_q_heads + kvh * G + h) * sg.mask_stride,
                             sg.tok_base + bs + lane);
#pragma unroll
            for (int i = 0; i < VPL; i++) o[h][i] *= alpha;
        }
        __syncthreads();
        for (int j = 0; j < nlive; j++) {
#pragma unroll
            for (int i = 0; i < VPL; i++) {
                const float vh = deq_v(ch, f, j, lane + 64 * i);
#pragma unroll
                for (int h = 0; h < G; h++) o[h][i] += ps[h][j] * vh;
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int h = 0; h < G; h++) {
        float* p = a.partials +
                   (((int64_t)b * a.num_q_heads + kvh * G + h) * a.total_splits + sg.split_base + sp) * (D + 2);
#pragma unroll
        for (int i = 0; i < VPL; i++) p[lane + 64 * i] = o[h][i];
        if (lane == 0) {
            p[D] = m[h];
            p[D + 1] = L[h];
        }
    }
}

template <int D>
static hipError_t launch_valu_d(const SplitArgs& a, int G, dim3 grid, hipStream_t st)
{
    switch (G) {
    case 1: hipLaunchKernelGGL((split_valu_kernel<D, 1>), grid, dim3(64), 0, st, a); break;
    case 2: hipLaunchKernelGGL((split_valu_kernel<D, 2>), grid, dim3(64), 0, st, a); break;
    case 4: hipLaunchKernelGGL((split_valu_kernel<D, 4>), grid, dim3(64), 0, st, a); break;
    case 8: hipLaunchKernelGGL((split_valu_kernel<D, 8>), grid, dim3(64), 0, st, a); break;
    case 16: hipLaunchKernelGGL((split_valu_kernel<D, 16>), grid, dim3(64), 0, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_split(const SegArgs& s, const void* q, int q_dtype, int32_t batch,
                               int32_t num_q_heads, float sm_scale, float tau_low,
                               int32_t split_tokens, int32_t total_splits, float* partials,
                               hipStream_t stream)
{
    if (batch == 0 || s.n_splits == 0) return hipSuccess;
    hipError_t err;
    if (launch_decode_split_mfma(s, q, q_dtype, batch, num_q_heads, sm_scale, tau_low, split_tokens, total_splits,
                                 partials, stream, &err))
        return err;
    if (launch_decode_split_f16(s, q, q_dtype, batch, num_q_heads, sm_scale, tau_low, split_tokens, total_splits,
                                partials, stream, &err))
        return err;
    SplitArgs a;
    a.seg = s;
    a.q = q;
    a.q_dtype = q_dtype;
    a.num_q_heads = num_q_heads;
    a.split_tokens = split_tokens;
    a.total_splits = total_splits;
    a.score_scale = sm_scale * 1.4426950408889634f;
    a.tau_low = tau_low;
    a.partials = partials;
    const int G = num_q_heads / s.f.H;
    dim3 grid((unsigned)s.n_splits, (unsigned)s.f.H, (unsigned)batch);
    return s.f.D == 64 ? launch_valu_d<64>(a, G, grid, stream) : launch_valu_d<128>(a, G, grid, stream);
}

// Merge of the split partials of one (sequence, query head), m in base 2:
//   M = max_i m_i,  O = sum_i o_i 2^(m_i - M) / sum_i L_i 2^(m_i - M).
// A split without tokens has m = -inf and an o row that was never written:
// its weight is 0 and its row is left out by a select (a stale NaN must not
// reach the sum).  One workgroup of NW waves per (sequence, query head): wave
// w merges splits [32 w, 32 w + 32), then [32 (w + NW), ...), loading each
// chunk's rows, maxima and sums together (one memory latency per chunk); with
// NW > 1 the running states are then merged through LDS.
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void combine_kernel(CombineArgs a)
{
    constexpr int VPL = D / 64;
    constexpr int CH = 32;
    const int64_t bh = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float* p = a.part + bh * a.total_splits * (D + 2);
    float acc[VPL];
#pragma unroll
    for (int j = 0; j < VPL; j++) acc[j] = 0.0f;
    float M = -INFINITY, L = 0.0f;
    for (int i0 = CH * wave; i0 < a.total_splits; i0 += CH * NW) {
        const int n = min(CH, a.total_splits - i0);
        float ov[CH][VPL];
#pragma unroll
        for (int i = 0; i < CH; i++) {
#pragma unroll
            for (int j = 0; j < VPL; j++) ov[i][j] = i < n ? p[(int64_t)(i0 + i) * (D + 2) + lane + 64 * j] : 0.0f;
        }
        const float mi = lane < n ? p[(int64_t)(i0 + lane) * (D + 2) + D] : -INFINITY;
        const float li = lane < n ? p[(int64_t)(i0 + lane) * (D + 2) + D + 1] : 0.0f;
        const float m_new = fmaxf(M, wave_max(mi));
        if (m_new == -INFINITY) continue;  // no token so far
        const float alpha = exp2f(M - m_new);
        const float wi = mi == -INFINITY ? 0.0f : exp2f(mi - m_new);
        L = L * alpha + wave_sum(li * wi);
#pragma unroll
        for (int j = 0; j < VPL; j++) acc[j] *= alpha;
#pragma unroll
        for (int i = 0; i < CH; i++) {
            const float w = __shfl(wi, i, 64);
#pragma unroll
            for (int j = 0; j < VPL; j++) acc[j] += w != 0.0f ? ov[i][j] * w : 0.0f;
        }
        M = m_new;
    }
    if constexpr (NW == 1) {
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
        for (int j = 0; j < VPL; j++) a.out[bh * D + lane + 64 * j] = acc[j] * inv;
        if (a.ml != nullptr && lane == 0) {
            a.ml[2 * bh] = M;
            a.ml[2 * bh + 1] = inv;
        }
        return;
    }
    // merge the waves' (M, L, acc)
    __shared__ float sm_m[NW], sm_l[NW];
    __shared__ float sm_o[NW][D];
    if (lane == 0) {
        sm_m[wave] = M;
        sm_l[wave] = L;
    }
#pragma unroll
    for (int j = 0; j < VPL; j++) sm_o[wave][lane + 64 * j] = acc[j];
    __syncthreads();
    if (wave != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; w++) Mt = fmaxf(Mt, sm_m[w]);
    float Lt = 0.0f, o[VPL];
#pragma unroll
    for (int j = 0; j < VPL; j++) o[j] = 0.0f;
    if (Mt != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; w++) {
            const float ww = sm_m[w] == -INFINITY ? 0.0f : exp2f(sm_m[w] - Mt);
            Lt += sm_l[w] * ww;
#pragma unroll
            for (int j = 0; j < VPL; j++) o[j] += sm_o[w][lane + 64 * j] * ww;
        }
    }
    const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
#pragma unroll
    for (int j = 0; j < VPL; j++) a.out[bh * D + lane + 64 * j] = o[j] * inv;
    if (a.ml != nullptr && lane == 0) {
        a.ml[2 * bh] = Mt;
        a.ml[2 * bh + 1] = inv;
    }
}

// The merge for head_dim 128 and at most CH (32 or 64) splits, the shape of
// the matrix-core decode: one wave per (sequence, query head) whose lane l
// holds channels 2l and 2l + 1 of every split's row (one 8-byte load per
// split) and split l's (m, L); merge128 does the arithmetic, as the split
// kernel that merges its own splits does.  Given the lengths, only the
// splits that hold tokens are read: the others' (m, L) are (-inf, 0), which
// is what the lanes past them take.  (Loads clamped to the last counted
// split and issued without branches measured no faster: at 32 splits the
// same, at 33 slower by the cache re-reads.)
template <int CH>
__global__ __launch_bounds__(64) void combine128_kernel(CombineArgs a)
{
    constexpr int D = 128;
    const int64_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    const float* p = a.part + bh * a.total_splits * (D + 2);
    int n = a.total_splits;
    if (a.lens != nullptr) {
        const int b = (int)(blockIdx.x / (unsigned)a.num_q_heads);
        const int len = max(0, min(a.lens[b], a.len_cap));
        n = min(n, (len + a.split_tokens - 1) / a.split_tokens);
    }
    float2 ov[CH];
#pragma unroll
    for (int i = 0; i < CH; i++) ov[i] = i < n ? *(const float2*)(p + (int64_t)i * (D + 2) + 2 * lane) : float2{};
    const float mi = lane < n ? p[(int64_t)lane * (D + 2) + D] : -INFINITY;
    const float li = lane < n ? p[(int64_t)lane * (D + 2) + D + 1] : 0.0f;
    float M, inv;
    *(float2*)(a.out + bh * D + 2 * lane) = merge128(ov, mi, li, &M, &inv);
    if (a.ml != nullptr && lane == 0) {
        a.ml[2 * bh] = M;
        a.ml[2 * bh + 1] = inv;
    }
}

// The merge for head_dim 128 with more than 32 splits: NW waves per
// (sequence, query head), each taking chunks of 32 splits in the layout of
// combine128_kernel (lane l: channels 2l and 2l + 1, one 8-byte load per
// split, weights by readlane), then the waves' (M, L, o) merged through
// LDS.  Per channel the same arithmetic, in the same order, as
// combine_kernel<128, NW>.
template <int NW>
__global__ __launch_bounds__(64 * NW) void combine128w_kernel(CombineArgs a)
{
    constexpr int D = 128, CH = 32;
    const int64_t bh = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float* p = a.part + bh * a.total_splits * (D + 2);
    float2 acc = {0.0f, 0.0f};
    float M = -INFINITY, L = 0.0f;
    for (int i0 = CH * wave; i0 < a.total_splits; i0 += CH * NW) {
        const int n = min(CH, a.total_splits - i0);
        float2 ov[CH];
#pragma unroll
        for (int i = 0; i < CH; i++)
            ov[i] = i < n ? *(const float2*)(p + (int64_t)(i0 + i) * (D + 2) + 2 * lane) : float2{};
        const float mi = lane < n ? p[(int64_t)(i0 + lane) * (D + 2) + D] : -INFINITY;
        const float li = lane < n ? p[(int64_t)(i0 + lane) * (D + 2) + D + 1] : 0.0f;
        const float m_new = fmaxf(M, wave_max(mi));
        if (m_new == -INFINITY) continue;  // no token so far
        const float alpha = exp2f(M - m_new);
        const float wi = mi == -INFINITY ? 0.0f : exp2f(mi - m_new);
        L = L * alpha + wave_sum(li * wi);
        acc.x *= alpha;
        acc.y *= alpha;
#pragma unroll
        for (int i = 0; i < CH; i++) {
            // splits past n have weight 0 (their lanes hold mi = -inf)
            const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wi), i));
            acc.x += w != 0.0f ? ov[i].x * w : 0.0f;
            acc.y += w != 0.0f ? ov[i].y * w : 0.0f;
        }
        M = m_new;
    }
    __shared__ float sm_m[NW], sm_l[NW];
    __shared__ float2 sm_o[NW][D / 2];
    if (lane == 0) {
        sm_m[wave] = M;
        sm_l[wave] = L;
    }
    sm_o[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    float Mt = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; w++) Mt = fmaxf(Mt, sm_m[w]);
    float Lt = 0.0f;
    float2 o = {0.0f, 0.0f};
    if (Mt != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; w++) {
            const float ww = sm_m[w] == -INFINITY ? 0.0f : exp2f(sm_m[w] - Mt);
            Lt += sm_l[w] * ww;
            o.x += sm_o[w][lane].x * ww;
            o.y += sm_o[w][lane].y * ww;
        }
    }
    const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
    *(float2*)(a.out + bh * D + 2 * lane) = float2{o.x * inv, o.y * inv};
    if (a.ml != nullptr && lane == 0) {
        a.ml[2 * bh] = Mt;
        a.ml[2 * bh + 1] = inv;
    }
}

hipError_t launch_decode_combine(const CombineArgs& a, int32_t batch, int32_t D, hipStream_t stream)
{
    if (batch == 0) return hipSuccess;
    const dim3 grid((unsigned)(batch * a.num_q_heads));
    // one wave takes up to 32 splits in one memory latency (at head_dim 128
    // up to 64, a split per lane); more splits are spread over four waves
    // (sixteen past 128 splits at head_dim 128)
    const bool one = a.total_splits <= 32;
    if (D == 64 && one) hipLaunchKernelGGL((combine_kernel<64, 1>), grid, dim3(64), 0, stream, a);
    else if (D == 64) hipLaunchKernelGGL((combine_kernel<64, 4>), grid, dim3(256), 0, stream, a);
    else if (one) hipLaunchKernelGGL(combine128_kernel<32>, grid, dim3(64), 0, stream, a);
    else if (a.total_splits <= 64) hipLaunchKernelGGL(combine128_kernel<64>, grid, dim3(64), 0, stream, a);
    else if (a.total_splits <= 4 * 32) hipLaunchKernelGGL(combine128w_kernel<4>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(combine128w_kernel<16>, grid, dim3(1024), 0, stream, a);
    return hipGetLastError();
}

// Accumulated attention scores: one thread per column of the score rows
// (a token of one segment) adds that token's softmax weight summed over the
// query heads, 2^(s - M) / L per head with the merged (M, 1 / L) of the head,
// to acc[segment][b][token].  Columns past a sequence's end were never
// written and are skipped.
__global__ __launch_bounds__(256) void score_accumulate_kernel(ScoreAccArgs a)
{
    const int b = blockIdx.y;
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= a.score_stride) return;
    const int seg = a.nseg > 1 && col >= a.tok_base[1] ? 1 : 0;
    const int j = col - a.tok_base[seg];
    const int len = max(0, min(a.lens[seg][b], a.len_cap[seg]));
    if (j >= len) return;
    const float* srow = a.scores + (int64_t)b * a.num_q_heads * a.score_stride + col;
    const float* ml = a.ml + (int64_t)b * a.num_q_heads * 2;
    // heads in groups of 4 whose loads are issued together
    float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int h = 0;
    for (; h + 4 <= a.num_q_heads; h += 4) {
        float x[4];
#pragma unroll
        for (int u = 0; u < 4; u++) x[u] = srow[(int64_t)(h + u) * a.score_stride];
#pragma unroll
        for (int u = 0; u < 4; u++) part[u] += exp2f(x[u] - ml[2 * (h + u)]) * ml[2 * (h + u) + 1];
    }
    for (; h < a.num_q_heads; h++) part[0] += exp2f(srow[(int64_t)h * a.score_stride] - ml[2 * h]) * ml[2 * h + 1];
    a.acc[((int64_t)seg * a.batch + b) * a.acc_stride + j] += (part[0] + part[1]) + (part[2] + part[3]);
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t stream)
{
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, v);
    return hipGetLastError();
}

hipError_t launch_score_accumulate(const ScoreAccArgs& a, hipStream_t stream)
{
    if (a.batch == 0 || a.score_stride == 0) return hipSuccess;
    const dim3 grid((unsigned)((a.score_stride + 255) / 256), (unsigned)a.batch);
    hipLaunchKernelGGL(score_accumulate_kernel, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lkv
