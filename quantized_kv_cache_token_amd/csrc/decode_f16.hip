// decode_f16.hip -- split-K decode attention with matrix cores over the
// fp16 cache of the sensitive layers (gfx950).
//
// The Super KV Compression page (first layer) keeps a few outlier layers in
// fp16.  Their chunks hold 64 fp16 K rows (token-major, 256 B each) and 128
// fp16 V rows (channel-major, 128 B each), four times the bytes of a K6V4
// chunk, so this kernel has one job: stream them at the memory rate.  Both
// products run on v_mfma_f32_16x16x32_f16 with the cache bytes as operands
// as loaded -- no unpacking at all.
//
// One wave owns one (split, KV head, sequence) and walks the split's blocks
// in order, 4 or 8 query heads per KV head, head_dim 128.
//
// Q.K: rows are 16 tokens, the K dimension is 32 channels, columns are
// (query head, part).  Q is multiplied by sm_scale log2(e) and by a power of
// two that brings the wave's largest |q| into [2^14, 2^15) (exact; no fp16
// overflow, no subnormal loss), then split into an fp16 high part and the
// fp16 rounding of the remainder, placed in the two columns of its head:
// the sum of the two columns is the score to about 22 significant bits.
//
// P.V: rows are (query head, part), the K dimension is 32 tokens, columns
// are 16 channels.  The weight p = 2^(s - m) <= 2^8 (the running maximum
// moves lazily, as in the K6 kernel) is scaled by 2^6 and split in the same
// way into the two rows of its head; the power of two is removed from the
// output at the end.
//
// Token order: QK tile t row m holds token 32 (t >> 1) + 8 (m >> 2) +
// 4 (t & 1) + (m & 3).  The four rows a lane receives from tiles 2u and 2u+1
// are then tokens 32u + 8 (l >> 4) + 0..7 in order, which is exactly its
// P.V A operand and matches the 16 contiguous V bytes it loads per channel.
//
// Online softmax, the sparse-V skip of the Super KV Compression page (third
// layer: after a block is folded into the running maximum m and sum L, a
// token with 2^(s - m) < tau_low L has its V term dropped) and the partial
// (o[128], m, L) per split are those of the generic kernel.
#include "lkv_internal.h"
#include "wave_util.h"

namespace lkv {

struct F16Args {
    SegArgs seg;
    const void* q;       // bf16 or fp32 [B][Hq][128]
    int32_t q_dtype;
    int32_t num_q_heads;
    int32_t split_tokens;
    int32_t total_splits;
    float score_scale;   // sm_scale * log2(e)
    float tau_low;
    float* partials;
};

constexpr int F16_D = 128;
constexpr int F16_KROW = 256;   // bytes of one K token row
constexpr int F16_VROW = 128;   // bytes of one V channel row
constexpr float P_SCALE = 64.0f;          // weights enter P.V as p * 2^6
constexpr float P_UNSCALE = 1.0f / 64.0f;

// Token of QK tile t (0..3), row m (0..15), within the 64-token block.
__device__ __forceinline__ constexpr int f16_tok(int t, int m)
{
    return 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3);
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi)
{
    const f16x2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// The part (0: fp16 high part, 1: fp16 rounding of the remainder) of x.
__device__ __forceinline__ float f16_part(float x, int part)
{
    const float hi = (float)(_Float16)x;
    return part ? x - hi : hi;
}

struct F16Block {
    uint4 k[4][4];   // K: tile t, K-step s -> channels 32s + 8(l>>4) + 0..7 of token f16_tok(t, l & 15)
    uint4 v[2][8];   // V: tile pair u, channel tile T -> tokens 32u + 8(l>>4) + 0..7 of channel 16T + (l & 15)
};

__device__ __forceinline__ void f16_load_k(F16Block& R, const uint8_t* ch, int c, int q)
{
#pragma unroll
    for (int t = 0; t < 4; t++) {
        const uint8_t* row = ch + f16_tok(t, c) * F16_KROW + 16 * q;
#pragma unroll
        for (int s = 0; s < 4; s++) R.k[t][s] = *(const uint4*)(row + 64 * s);
    }
}

__device__ __forceinline__ void f16_load_v(F16Block& R, const uint8_t* ch, uint32_t off_vc, int c, int q)
{
#pragma unroll
    for (int u = 0; u < 2; u++) {
#pragma unroll
        for (int T = 0; T < 8; T++) R.v[u][T] = *(const uint4*)(ch + off_vc + (16 * T + c) * F16_VROW + 64 * u + 16 * q);
    }
}

__device__ __forceinline__ void as_words(const uint4& x, uint32_t (&w)[4])
{
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
}

// DBG: the same kernel that also records its skip decisions (the test entry
// point's skip mask); production launches take DBG = false.
template <int G, bool DBG>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void split_f16_kernel(F16Args a)
{
    static_assert(G == 4 || G == 8, "4 or 8 query heads per KV head");
    constexpr int D = F16_D;
    const SegArgs& sg = a.seg;
    const Fmt& f = sg.f;
    const int sp = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int c = lane & 15, q = lane >> 4;
    const int t0 = sp * a.split_tokens;
    // the split's block-table entries (at most 64, one per lane) do not
    // depend on the length: they are requested together with it
    // (the sequence and length are uniform: computed before the lane-dependent
    // load, so that they stay in scalar registers)
    const int seq = entry_seq(sg, b);
    const int len = max(0, min(entry_len(sg, b), sg.len_cap));
    const int32_t* bt = sg.block_table + (int64_t)seq * sg.max_blocks + t0 / BT;
    const int bt_lane = lane < min(64, sg.max_blocks - t0 / BT) ? bt[lane] : 0;
    asm volatile("" ::: "memory");  // both loads are issued before either is waited for
    const int t1 = min(t0 + a.split_tokens, len);
    if (t1 <= t0) {  // a split past the end: only (m, L) = (-inf, 0), its o row is never read
        if (threadIdx.x < G) {
            float* p = a.partials + (((int64_t)b * a.num_q_heads + kvh * G + threadIdx.x) * a.total_splits +
                                     sg.split_base + sp) * (D + 2);
            p[D] = -INFINITY;
            p[D + 1] = 0.0f;
        }
        return;
    }

    // QK column / P.V row c -> (head hc, part c & 1); with G = 4, columns
    // and rows 8..15 repeat 0..7.
    const int hc = (c & (2 * G - 1)) >> 1;
    const int part = c & 1;
    const int head = kvh * G + hc;
    // heads of the P.V output rows this lane holds (rows 4q .. 4q+3)
    const int hA = G == 8 ? 2 * q : 2 * (q & 1);
    // this lane's head's score row, at the split's first token; the part-0
    // lane of each head stores the scores when the call asks for them
    float* const srow = sg.scores != nullptr && part == 0 && c < 2 * G
                            ? sg.scores + ((int64_t)b * a.num_q_heads + head) * sg.score_stride + sg.tok_base + t0
                            : nullptr;
    // the same lane's skip-mask row (test entry point only)
    uint32_t* const mrow = DBG && sg.skip_mask != nullptr && part == 0 && c < 2 * G
                               ? sg.skip_mask + ((int64_t)b * a.num_q_heads + head) * sg.mask_stride
                               : nullptr;

    // ---- Q as the QK B operand: K-step s, K index 8q + i <-> channel 32s + 8q + i
    float x[4][8];
    {
        const int64_t qrow = ((int64_t)b * a.num_q_heads + head) * D;
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int d0 = 32 * s + 8 * q;
            if (a.q_dtype == LKV_BF16) {
                const uint4 w = *(const uint4*)((const uint16_t*)a.q + qrow + d0);
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    x[s][2 * i] = __uint_as_float(ww[i] << 16);
                    x[s][2 * i + 1] = __uint_as_float(ww[i] & 0xFFFF0000u);
                }
            } else {
                const float4 w0 = *(const float4*)((const float*)a.q + qrow + d0);
                const float4 w1 = *(const float4*)((const float*)a.q + qrow + d0 + 4);
                x[s][0] = w0.x; x[s][1] = w0.y; x[s][2] = w0.z; x[s][3] = w0.w;
                x[s][4] = w1.x; x[s][5] = w1.y; x[s][6] = w1.z; x[s][7] = w1.w;
            }
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; s++) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            x[s][i] *= a.score_scale;
            amax = fmaxf(amax, fabsf(x[s][i]));
        }
    }
    for (int o = 1; o < 64; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    // 2^e > amax >= 2^(e-1): scale by 2^(15 - e); scores come out times that
    const int e = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) : 0;
    const int qexp = 15 - e;
    const float unscale = __builtin_amdgcn_ldexpf(1.0f, -qexp);
    uint32_t qb[4][4];
#pragma unroll
    for (int s = 0; s < 4; s++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float y0 = __builtin_amdgcn_ldexpf(x[s][2 * i], qexp);
            const float y1 = __builtin_amdgcn_ldexpf(x[s][2 * i + 1], qexp);
            qb[s][i] = pack_f16(f16_part(y0, part), f16_part(y1, part));
        }
    }

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4_t acc[8];
#pragma unroll
    for (int T = 0; T < 8; T++) acc[T] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int nblk = (t1 - t0 + BT - 1) / BT;
    const uint8_t* const pool = sg.pool;
    const int64_t chunk = f.chunk;
    const int H = f.H;
    const uint32_t off_vc = (uint32_t)f.off_vc;
    auto chunk_of = [=](int k) {
        const int blk = __builtin_amdgcn_readlane(bt_lane, k);
        return pool + ((int64_t)blk * H + kvh) * chunk;
    };

    F16Block R;
    {
        const uint8_t* c0 = chunk_of(0);
        f16_load_k(R, c0, c, q);
        asm volatile("" ::: "memory");
        f16_load_v(R, c0, off_vc, c, q);
        asm volatile("" ::: "memory");
    }
    // (the empty asm statements keep the compiler from moving the next
    // block's loads to their first use)
    for (int k = 0; k < nblk; k++) {
        const uint8_t* cn = chunk_of(min(k + 1, nblk - 1));
        const int nlive = min(BT, t1 - t0 - k * BT);

        // ---- Q.K: 4 tiles x 4 K-steps
        f32x4_t dot[4];
#pragma unroll
        for (int t = 0; t < 4; t++) {
            f32x4_t d4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; s++) {
                uint32_t ka[4];
                as_words(R.k[t][s], ka);
                d4 = mfma_16x16x32_f16(ka, qb[s], d4);
            }
            dot[t] = d4;
        }
        f16_load_k(R, cn, c, q);
        asm volatile("" ::: "memory");

        // ---- scores of the lane's 16 tokens (p index 4t + r), online softmax
        float p[16];
        float bmax = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; t++) {
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float d = dot[t][r];
                float s2 = (d + xor1(d)) * unscale;  // both parts of the head, base 2
                if (nlive < BT) s2 = f16_tok(t, 4 * q + r) < nlive ? s2 : -INFINITY;
                p[4 * t + r] = s2;
                bmax = fmaxf(bmax, s2);
            }
        }
        if (srow != nullptr) {
            // tokens f16_tok(t, 4q) .. + 3 of tile t are consecutive
            float* dst = srow + (int64_t)k * BT;
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const int x = f16_tok(t, 4 * q);
                if (nlive == BT) {
                    *(float4*)(dst + x) = make_float4(p[4 * t], p[4 * t + 1], p[4 * t + 2], p[4 * t + 3]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        if (x + r < nlive) dst[x + r] = p[4 * t + r];
                }
            }
        }
        bmax = rows_max(bmax);
        const float m_new = bmax > m_run + 8.0f ? bmax : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float bsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            p[i] = __builtin_amdgcn_exp2f(p[i] - m_new);
            bsum += p[i];
        }
        l_run = l_run * alpha + rows_sum(bsum);
        m_run = m_new;
        uint32_t keep = 3u;
        if (a.tau_low > 0.0f) {  // sparse-V skip against the running bound
            const float thr = a.tau_low * l_run;
            bool k0 = false, k1 = false;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                p[i] = p[i] < thr ? 0.0f : p[i];
                if (i < 8) k0 |= p[i] > 0.0f;   // tiles 0, 1: P.V tile pair 0
                else k1 |= p[i] > 0.0f;
            }
            keep = (__builtin_amdgcn_ballot_w64(k0) ? 1u : 0u) | (__builtin_amdgcn_ballot_w64(k1) ? 2u : 0u);
            if (mrow != nullptr) {  // a live token's weight is 0 here exactly when it was below thr
#pragma unroll
                for (int t = 0; t < 4; t++) {
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        const int x = f16_tok(t, 4 * q + r);
                        if (x < nlive && p[4 * t + r] == 0.0f) mark_skipped(mrow, sg.tok_base + t0 + k * BT + x);
                    }
                }
            }
        }

        // ---- P.V
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
            const float alA = __shfl(alpha, 2 * hA, 64), alB = __shfl(alpha, 2 * hA + 2, 64);
#pragma unroll
            for (int T = 0; T < 8; T++) {
                acc[T][0] *= alA;
                acc[T][1] *= alA;
                acc[T][2] *= alB;
                acc[T][3] *= alB;
            }
        }
        if (nlive < BT) {
            // V of tokens past the end may hold any bits (a NaN would reach
            // every head through the product): zero them
#pragma unroll
            for (int u = 0; u < 2; u++) {
                uint32_t msk[4];
#pragma unroll
                for (int w = 0; w < 4; w++) {
                    const int tok = 32 * u + 8 * q + 2 * w;
                    msk[w] = (tok < nlive ? 0x0000FFFFu : 0u) | (tok + 1 < nlive ? 0xFFFF0000u : 0u);
                }
#pragma unroll
                for (int T = 0; T < 8; T++) {
                    R.v[u][T].x &= msk[0];
                    R.v[u][T].y &= msk[1];
                    R.v[u][T].z &= msk[2];
                    R.v[u][T].w &= msk[3];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 2; u++) {
            if (!(keep & (1u << u))) continue;  // every V term of the 32 tokens skipped
            uint32_t pa[4];
#pragma unroll
            for (int i = 0; i < 4; i++)
                pa[i] = pack_f16(f16_part(p[8 * u + 2 * i] * P_SCALE, part),
                                 f16_part(p[8 * u + 2 * i + 1] * P_SCALE, part));
#pragma unroll
            for (int T = 0; T < 8; T++) {
                uint32_t bv[4];
                as_words(R.v[u][T], bv);
                acc[T] = mfma_16x16x32_f16(pa, bv, acc[T]);
            }
        }
        f16_load_v(R, cn, off_vc, c, q);
        asm volatile("" ::: "memory");
    }

    // ---- write the partial (o, m, L) of every head of the group
    float* base = a.partials + ((int64_t)b * a.num_q_heads + kvh * G) * a.total_splits * (D + 2);
    const int64_t hstride = (int64_t)a.total_splits * (D + 2);
    const int64_t soff = (int64_t)(sg.split_base + sp) * (D + 2);
    if (G == 8 || q < 2) {
#pragma unroll
        for (int T = 0; T < 8; T++) {
            base[hA * hstride + soff + 16 * T + c] = (acc[T][0] + acc[T][1]) * P_UNSCALE;
            base[(hA + 1) * hstride + soff + 16 * T + c] = (acc[T][2] + acc[T][3]) * P_UNSCALE;
        }
    }
    if (q == 0 && part == 0 && (G == 8 || c < 8)) {
        base[hc * hstride + soff + D] = m_run;
        base[hc * hstride + soff + D + 1] = l_run;
    }
}

bool launch_decode_split_f16(const SegArgs& s, const void* q, int q_dtype, int32_t batch, int32_t num_q_heads,
                             float sm_scale, float tau_low, int32_t split_tokens, int32_t total_splits,
                             float* partials, hipStream_t stream, hipError_t* err)
{
    const Fmt& f = s.f;
    const int G = num_q_heads / f.H;
    if (!f.fp16 || f.D != F16_D || (q_dtype != LKV_BF16 && q_dtype != LKV_F32) || (G != 4 && G != 8) ||
        ((uintptr_t)q & 15) != 0)  // Q is read 16 bytes at a time
        return false;
    if (split_tokens > 64 * BT) return false;  // a split's block-table entries are held one per lane
    F16Args a;
    a.seg = s;
    a.q = q;
    a.q_dtype = q_dtype;
    a.num_q_heads = num_q_heads;
    a.split_tokens = split_tokens;
    a.total_splits = total_splits;
    a.score_scale = sm_scale * 1.4426950408889634f;
    a.tau_low = tau_low;
    a.partials = partials;
    dim3 grid((unsigned)s.n_splits, (unsigned)f.H, (unsigned)batch);
    const bool dbg = s.skip_mask != nullptr;
    if (G == 4 && dbg) hipLaunchKernelGGL((split_f16_kernel<4, true>), grid, dim3(64), 0, stream, a);
    else if (G == 4) hipLaunchKernelGGL((split_f16_kernel<4, false>), grid, dim3(64), 0, stream, a);
    else if (dbg) hipLaunchKernelGGL((split_f16_kernel<8, true>), grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL((split_f16_kernel<8, false>), grid, dim3(64), 0, stream, a);
    *err = hipGetLastError();
    return true;
}

}  // namespace lkv
