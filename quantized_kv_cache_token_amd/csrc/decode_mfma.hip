// decode_mfma.hip -- split-K decode attention with matrix cores (gfx950).
//
// For bf16 queries over a K6 cache (V4 or V6), head_dim 128, group 64, and 4
// or 8 query heads per KV head.  One wave owns one (split, KV head,
// sequence); a split walks its 64-token blocks in order, 16-token tiles at a
// time.
//
// Q.K (v_mfma_f32_16x16x32_bf16): rows are tokens, columns are (query head,
// channel group) pairs, so one MFMA produces the per-group dot products
//   dot'(t, h, g) = sum_{d in g} q_hd * (128 + c_td)
// where the bf16 A operand is built from the 6-bit code c by placing it in
// the mantissa of 128.0 (exact); Q is the B operand, masked to the group.
// With 4 query heads per KV head (one query token) the K dimension of each
// product carries two 16-token sets instead, and the columns are (set, head,
// group): every column is used and a lane scores 8 tokens of a block, not 16
// (the two-set layout below).
// The score of a token is then
//   s(t, h) = sm * sum_g s_g(t) * (dot'(t, h, g) - (128 + z_g(t)) * qsum(h, g))
// with qsum(h, g) the sum of q over the group, i.e. the dequantised dot
// product sum_d q_hd (c_td - z) s.  Scores are kept in base-2 units.
//
// P.V (v_mfma_f32_16x16x32_bf16, 32 tokens): rows are (query head, hi/lo part),
// the K dimension is tokens, columns are channels.  The A operand carries
// p'(t) = p(t) * s_v(t) split into a bf16 high part and the bf16 rounding
// of the remainder (16 significant bits together); the B operand carries
// OFF + c (OFF = 128 for 6-bit codes and for the first nibble pair of a
// 4-bit word, 16 for its other pairs; all exact in bf16).  sum_t p'(t) (OFF + z(t)) is accumulated beside it and subtracted
// at the end, giving sum_t p(t) s_v(t) (c_t - z(t)) = sum_t p(t) v_hat(t).
//
// The QK result registers of a lane are exactly the P.V A-operand registers
// it needs (rows of the QK output = K index of the P.V input), so no data
// moves between the two products.  Token order inside a block is permuted
// (the same permutation on both sides) so that the V bytes a lane loads
// unpack with one shift and one mask per pair of 4-bit codes.
//
// Online softmax per head, the sparse-V skip of the Super KV Compression
// page (third layer: after a block is folded into the running maximum m and
// sum L, exp(s - m) < tau_low * L drops the token's V term) and the partial
// (o[128], m, L) per split follow the generic kernel exactly.
#include <hip/hip_fp16.h>

#include <type_traits>

#include "lkv_internal.h"
#include "merge128.h"
#include "quant_device.h"
#include "wave_util.h"

namespace lkv {

struct MfmaArgs {
    SegArgs seg;
    const uint16_t* q;   // bf16 [B][Hq][128]
    int32_t num_q_heads;
    int32_t split_tokens;
    int32_t total_splits;
    float score_scale;   // sm_scale * log2(e)
    float tau_low;
    float* partials;
    // the step's new K and V rows [B][Hkv][128] (lkv_append_decode), in kv_dtype
    const void* k_new;
    const void* v_new;
    int32_t kv_dtype;
    // the split kernel that merges its own splits: one counter per (entry, KV
    // head) row, zero between calls, and the output [B][Hq][128]
    uint32_t* counters;
    float* out;
    // multi-token calls with 8 query heads per KV head: (split, KV head,
    // sequence) items, each run for the call's T query tokens
    int32_t items;
    // the decode step of a ragged batch of at most 64 sequences: its entry
    // count, and the grid in compact order (split_append_kernel); 0 otherwise
    int32_t compact;
};

// The bit manipulations below are plain C, never inline asm: a matrix-core
// instruction that reads a VGPR just written by a vector instruction needs
// wait states, which the compiler inserts only for instructions it can see.
// (An asm block feeding an MFMA operand one instruction later gave wrong
// products under some schedules.)

// x | (x << 10) (v_lshl_or_b32).
__device__ __forceinline__ uint32_t lshl10_or(uint32_t x) { return (x << 10) | x; }

// (x & m) | c (v_and_or_b32).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) { return (x & m) | c; }

// Constants of the code-to-bf16 conversions, kept in registers.
struct Magic {
    uint32_t m6, c6;   // 0x003F003F, 0x43004300: 6-bit code -> 128 + c
    uint32_t m4, c4;   // 0x00780078, 0x41804180: 4-bit code (at bit 3) -> 16 + c
    uint32_t m4lo;     // 0x000F000F: 4-bit code at bit 0 -> 128 + c (with c6)
};

// v in a VGPR, its value hidden from the optimiser so that the constants
// stay in registers and (x & m) | c is one v_and_or_b32 rather than two
// instructions with literals.  The asm holds no instruction: the v_mov that
// sets the register is the compiler's own.
__device__ __forceinline__ uint32_t opaque(uint32_t v)
{
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ Magic make_magic()
{
    return Magic{opaque(0x003F003Fu), opaque(0x43004300u), opaque(0x00780078u), opaque(0x41804180u),
                 opaque(0x000F000Fu)};
}

// Two adjacent 6-bit codes at bit BIT of an N-word bitstream, as a pair of
// bf16 values 128 + c (low half: the first code).
template <int BIT, int N>
__device__ __forceinline__ uint32_t pair6(const uint32_t (&w)[N], const Magic& k)
{
    constexpr int wi = BIT >> 5, sh = BIT & 31;
    uint32_t x;
    if constexpr (sh <= 20) {
        x = __builtin_amdgcn_ubfe(w[wi], sh, 12);
    } else {
        x = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & 0xFFFu;
    }
    return and_or(lshl10_or(x), k.m6, k.c6);  // code a at bits 0..5, code b at 16..21
}

// K codes, 16 at a time (96 bits, 3 words; code k at bits 6k).  Any pairing
// of channels into bf16 pairs works as long as Q uses the same one, so codes
// are paired by position: twelve of the sixteen lie inside a 16-bit half and
// pair up as (low-half code, high-half code) of one word, unpacked by one
// packed 16-bit shift and one and_or; the four that straddle a half pair up
// as (2, 13) and (5, 10).  Pair j of group n covers channels
//   KPAIR[j] = {(0,3), (1,4), (6,8), (7,9), (11,14), (12,15), (2,13), (5,10)}.
// Both 16-bit halves of w shifted right by the matching half of sh (each
// below 16) (v_pk_lshrrev_b16).
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_shr(uint32_t w, uint32_t sh)
{
    const u16x2_t r = __builtin_bit_cast(u16x2_t, w) >> __builtin_bit_cast(u16x2_t, sh);
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ void k16_pairs(uint32_t w0, uint32_t w1, uint32_t w2, const Magic& k, uint32_t (&o)[8])
{
    o[0] = and_or(pk_shr(w0, 0x00020000u), k.m6, k.c6);  // codes 0 (lo >> 0), 3 (hi >> 2)
    o[1] = and_or(pk_shr(w0, 0x00080006u), k.m6, k.c6);  // codes 1, 4
    o[2] = and_or(pk_shr(w1, 0x00000004u), k.m6, k.c6);  // codes 6, 8
    o[3] = and_or(pk_shr(w1, 0x0006000Au), k.m6, k.c6);  // codes 7, 9
    o[4] = and_or(pk_shr(w2, 0x00040002u), k.m6, k.c6);  // codes 11, 14
    o[5] = and_or(pk_shr(w2, 0x000A0008u), k.m6, k.c6);  // codes 12, 15
    // code 2 = bits 12..17 of w0, code 13 = bits 14..19 of w2
    o[6] = and_or(__builtin_amdgcn_perm(w2 << 2, w0 >> 12, 0x07060100u), k.m6, k.c6);
    // code 5 = bits 30..35, code 10 = bits 60..65 of the stream
    o[7] = and_or(__builtin_amdgcn_perm(__builtin_amdgcn_alignbit(w2, w1, 28), __builtin_amdgcn_alignbit(w1, w0, 30),
                                        0x05040100u),
                  k.m6, k.c6);
}

// Channel (0..15 of a 16-channel group) of element e (0 = low half) of
// K pair j.
__device__ __forceinline__ constexpr int kpair_ch(int j, int e)
{
    constexpr int a[8] = {0, 1, 6, 7, 11, 12, 2, 5};
    constexpr int b[8] = {3, 4, 8, 9, 14, 15, 13, 10};
    return e == 0 ? a[j] : b[j];
}

// Nibbles K and K+4 of w as a pair of bf16 values: OFF4<K> + c.  Nibbles 0
// and 4 already sit in the low mantissa bits of the two halves and become
// 128 + c with no shift; the others are shifted to bit 3 and become 16 + c.
template <int K>
__device__ __forceinline__ uint32_t pair4(uint32_t w, const Magic& k)
{
    if constexpr (K == 0) return and_or(w, k.m4lo, k.c6);
    else return and_or(w >> (4 * K - 3), k.m4, k.c4);
}

// Token (0..15 of the lane group's 16) of row r of QK tile t.  4-bit V: the
// rows of tiles 2u, 2u+1 are nibbles (0,4,1,5 | 2,6,3,7) of one V word, so
// the P.V K index j of tile pair u is nibble {0,4,1,5,2,6,3,7}[j]; 6-bit V:
// natural order.
template <int VB>
__device__ __forceinline__ constexpr int tok_of(int t, int r)
{
    if constexpr (VB == 4) {
        // nibble {0,4,1,5}[r] of word t>>1 for even t, {2,6,3,7}[r] for odd t
        return 8 * (t >> 1) + 2 * (t & 1) + (r >> 1) + 4 * (r & 1);
    } else {
        return 4 * t + r;
    }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest-even bf16, packed low/high.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// a * b rounded to fp32 on its own: never fused into a later addition.
__device__ __forceinline__ float mul_rounded(float a, float b)
{
#pragma clang fp contract(off)
    return a * b;
}

__device__ __forceinline__ uint32_t byte_of(const uint32_t (&w)[4], int x) { return (w[x >> 2] >> (8 * (x & 3))) & 0xFFu; }

// Raw bytes of one block held by one lane: codes in registers, the block's
// scales and zero points (1280 contiguous bytes: K scales, V scales, K zeros,
// V zeros) through a per-wave LDS buffer.
template <int VB>
struct BlockRegs {
    uint32_t kr[4][6];                  // K: tile t -> 32 channels of one token
    uint32_t vr[8][VB == 4 ? 2 : 3];    // V: channel tile T -> 16 tokens of one channel
    uint4 meta[2];                      // this lane's 16 B slices of the metadata
};

constexpr int META_BYTES = 1280;        // D 128, group 64: 2 groups x 64 slots x (4 + 4 + 1 + 1)
// With direction-preserving K the 64 fp32 norm factors follow at once
// (every section is a multiple of 128 B): 1536 contiguous bytes.
constexpr int META_KN_BYTES = META_BYTES + 256;
template <bool KN> constexpr int meta_bytes() { return KN ? META_KN_BYTES : META_BYTES; }
constexpr int META_VS = 512, META_KZ = 1024, META_VZ = 1152;

// Cache loads.  Every byte of the cache is read once per call.  The V codes
// and the metadata are read with non-temporal loads (global_load ... nt):
// each of those instructions consumes whole 128-byte lines, and on this part
// that raises the streaming read rate of a decode-shaped pass from about 5.7
// to 6.4 TB/s.  The K loads stay ordinary: a lane's 24 bytes of a 96-byte
// row take two instructions that touch the same lines, and with the
// non-temporal hint the second touch went back to HBM (the kernel ran
// slower).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 ld_nt(const uint2* p)
{
    const u32x2_t v = __builtin_nontemporal_load((const u32x2_t*)p);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 ld_nt(const uint4* p)
{
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }

template <int VB>
__device__ __forceinline__ void load_k(BlockRegs<VB>& R, const uint8_t* ch, uint32_t off_kc, int c, int q)
{
#pragma unroll
    for (int t = 0; t < 4; t++) {
        const uint32_t tok = 16 * (c >> 2) + tok_of<VB>(t, c & 3);
        const uint2* p = (const uint2*)(ch + (off_kc + tok * 96 + 24 * q));
        const uint2 x0 = p[0], x1 = p[1], x2 = p[2];
        R.kr[t][0] = x0.x; R.kr[t][1] = x0.y; R.kr[t][2] = x1.x;
        R.kr[t][3] = x1.y; R.kr[t][4] = x2.x; R.kr[t][5] = x2.y;
    }
}

template <int VB>
__device__ __forceinline__ void load_v(BlockRegs<VB>& R, const uint8_t* ch, uint32_t off_vc, int c, int q)
{
#pragma unroll
    for (int T = 0; T < 8; T++) {
        if constexpr (VB == 4) {
            const uint2 x = ld_nt((const uint2*)(ch + (off_vc + (16 * T + c) * 32 + 8 * q)));
            R.vr[T][0] = x.x;
            R.vr[T][1] = x.y;
        } else {
            const uint32_t* p = (const uint32_t*)(ch + (off_vc + (16 * T + c) * 48 + 12 * q));
            R.vr[T][0] = ld_nt(p);
            R.vr[T][1] = ld_nt(p + 1);
            R.vr[T][2] = ld_nt(p + 2);
        }
    }
}

template <int VB, bool KN>
__device__ __forceinline__ void load_meta(BlockRegs<VB>& R, const uint8_t* ch, uint32_t off_ks, int lane)
{
    const uint4* m = (const uint4*)(ch + off_ks);
    R.meta[0] = ld_nt(m + lane);
    R.meta[1] = ld_nt(m + 64 + min(lane, (meta_bytes<KN>() - 1024) / 16 - 1));  // every lane loads: no branch
}

template <bool KN>
__device__ __forceinline__ void stage_meta(const uint4 (&meta)[2], uint4* lds, int lane)
{
    lds[lane] = meta[0];
    // lanes past the last slice rewrite it with the same bytes: no branch
    lds[64 + min(lane, (meta_bytes<KN>() - 1024) / 16 - 1)] = meta[1];
}

__device__ __forceinline__ void read16f(const uint8_t* lds, float (&v)[16])
{
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const float4 x = ((const float4*)lds)[i];
        v[4 * i] = x.x; v[4 * i + 1] = x.y; v[4 * i + 2] = x.z; v[4 * i + 3] = x.w;
    }
}

__device__ __forceinline__ void read16b(const uint8_t* lds, uint32_t (&w)[4])
{
    const uint4 x = *(const uint4*)lds;
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
}

// Running state of one lane.
struct SplitState {
    float m_run, l_run;
    f32x4_t acc[8];
};

// One 64-token block in three phases (the kernel issues the next block's
// loads between them): Q.K, scores + online softmax + sparse-V skip, P.V.
template <int VB>
__device__ __forceinline__ void block_qk(const BlockRegs<VB>& R, const uint32_t (&qb)[4][4], float q128,
                                         const Magic& mk, f32x4_t (&dot)[4])
{
    // ---- Q.K: 4 tiles x 4 K-steps of 8 channel pairs
#pragma unroll
    for (int t = 0; t < 4; t++) {
        uint32_t ka[4][4];
        uint32_t lo[8], hi[8];
        k16_pairs(R.kr[t][0], R.kr[t][1], R.kr[t][2], mk, lo);
        k16_pairs(R.kr[t][3], R.kr[t][4], R.kr[t][5], mk, hi);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            ka[0][j] = lo[j];
            ka[1][j] = lo[4 + j];
            ka[2][j] = hi[j];
            ka[3][j] = hi[4 + j];
        }
        f32x4_t d4 = {-q128, -q128, -q128, -q128};  // removes the 128 offset of the codes
#pragma unroll
        for (int s = 0; s < 4; s++) d4 = mfma_16x16x32(ka[s], qb[s], d4);
        dot[t] = d4;
    }

}

// 8-head layout (8 heads of one token, or 4 heads of each of a query-token
// pair): scores of the lane's 16 tokens from the block's dot products, folded into
// the running (m, L); fills the weights p (0 for dead or skipped tokens) and
// returns the rescale factor of this lane's head.  keep: bit u set unless
// every V term of tile pair u (32 tokens) is skipped for every head.
// PARTIAL: the block has dead slots past the end (nlive < 64), masked here;
// full blocks skip that work.  score_scale > 0 is applied after the maximum
// (the maximum of scaled scores is the scaled maximum), inside the exponent.
// srow: when non-null, the block's column of this lane's head in the score
// rows; the lane that owns the head (part 0) stores its 16 tokens' base-2
// scores there.
template <int VB, bool PARTIAL, bool KN>
__device__ __forceinline__ float block_softmax(const f32x4_t (&dot)[4], const uint8_t* lds, SplitState& S, float qsum,
                                               float score_scale, float tau_low, int nlive, int q, int c,
                                               float (&p)[16], uint32_t& keep, float* srow, uint32_t* mrow,
                                               int mcol)
{
    const int gc = c & 1;
    float sk[16];
    uint32_t zk[4];
    read16f(lds + gc * 256 + 64 * q, sk);
    read16b(lds + META_KZ + gc * 64 + 16 * q, zk);
    float sc[16];
    float rk[16];  // direction-preserving K: the norm factors of the lane's 16 tokens
    if constexpr (KN) read16f(lds + META_BYTES + 64 * q, rk);
    float bmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; t++) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int x = tok_of<VB>(t, r);
            // this lane's group share: s_g * sum_{d in g} q_d (c_d - z_g),
            // rounded before the exchange so that the two lanes of a head
            // add the same two numbers and hold bit-identical scores (their
            // running maxima must never differ)
            const float pg = mul_rounded(sk[x], dot[t][r] - (float)byte_of(zk, x) * qsum);
            float s2 = pg + xor1(pg);  // both groups, natural units
            if constexpr (KN) s2 *= rk[x];  // the key is r * k_hat (the same product on both lanes)
            if constexpr (PARTIAL) s2 = 16 * q + x < nlive ? s2 : -INFINITY;
            sc[4 * t + r] = s2;
            bmax = fmaxf(bmax, s2);
        }
    }
    if (srow != nullptr && (c & 1) == 0) {
        float v[16];  // token 16 q + i of the block
#pragma unroll
        for (int t = 0; t < 4; t++) {
#pragma unroll
            for (int r = 0; r < 4; r++) v[tok_of<VB>(t, r)] = sc[4 * t + r] * score_scale;
        }
        float* dst = srow + 16 * q;
        if constexpr (PARTIAL) {
#pragma unroll
            for (int i = 0; i < 16; i++)
                if (16 * q + i < nlive) dst[i] = v[i];
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) ((float4*)dst)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        }
    }
    bmax = rows_max(bmax) * score_scale;  // base 2
    // The reference maximum only moves when a block exceeds it by more than
    // 2^8: weights stay <= 256 (no overflow anywhere), the accumulators are
    // rarely rescaled, and p / L -- all that the output and the skip rule
    // depend on -- does not change.
    const float m_new = bmax > S.m_run + 8.0f ? bmax : S.m_run;
    // a masked block can leave a column with no live token so far (the
    // earlier token of a query pair): its weights are 0, not exp2(NaN)
    const float m_ref = PARTIAL && m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(S.m_run - m_ref);
    float bsum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], score_scale, -m_ref));
        bsum += p[i];
    }
    S.l_run = S.l_run * alpha + rows_sum(bsum);
    S.m_run = m_new;
    keep = 3u;
    if (tau_low > 0.0f) {  // sparse-V skip against the running bound
        const float thr = tau_low * S.l_run;
        bool k0 = false, k1 = false;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            p[i] = p[i] < thr ? 0.0f : p[i];
            if (i < 8) k0 |= p[i] > 0.0f;   // tiles 0, 1: P.V tile pair 0
            else k1 |= p[i] > 0.0f;
        }
        keep = (__builtin_amdgcn_ballot_w64(k0) ? 1u : 0u) | (__builtin_amdgcn_ballot_w64(k1) ? 2u : 0u);
        if (mrow != nullptr && (c & 1) == 0) {  // a live token's weight is 0 here exactly when it was below thr
#pragma unroll
            for (int t = 0; t < 4; t++) {
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int tok = 16 * q + tok_of<VB>(t, r);
                    if ((!PARTIAL || tok < nlive) && p[4 * t + r] == 0.0f) mark_skipped(mrow, mcol + tok);
                }
            }
        }
    }
    return alpha;
}

// bf16 pairs of -(OFF + z) for the 8 tokens of P.V tile pair u (K index j
// = 2k, 2k+1 in pair k), from the zero-point bytes of the lane's 16 tokens.
template <int VB>
__device__ __forceinline__ void neg_off_pairs(const uint32_t (&z)[4], int u, uint32_t (&o)[4])
{
    const uint32_t lo = z[2 * u], hi = z[2 * u + 1];  // tokens 8u .. 8u+3, 8u+4 .. 8u+7
#pragma unroll
    for (int k = 0; k < 4; k++) {
        if constexpr (VB == 4) {
            // K index 2k, 2k+1 are tokens 8u + k, 8u + k + 4: byte k of lo and of hi
            const uint32_t x = __builtin_amdgcn_perm(hi, lo, 0x0C000C00u | (uint32_t)k | ((uint32_t)(4 + k) << 16));
            o[k] = k == 0 ? x | 0xC300C300u : (x << 3) | 0xC180C180u;  // -(OFF4<k> + z): 128 for k = 0, else 16
        } else {
            // K index 2k, 2k+1 are tokens 8u + 2k, 8u + 2k + 1
            const uint32_t w = k < 2 ? lo : hi;
            const uint32_t b0 = (uint32_t)(2 * (k & 1));
            const uint32_t x = __builtin_amdgcn_perm(w, w, 0x0C000C00u | b0 | ((b0 + 1) << 16));
            o[k] = x | 0xC300C300u;  // -(128 + z)
        }
    }
}

// 8-head layout: P.V of the block, rows (head, part); each V group has an
// A operand of its own.
template <int VB, bool PARTIAL>
__device__ __forceinline__ void block_pv(const BlockRegs<VB>& R, const uint8_t* lds, SplitState& S,
                                         const float (&p)[16], float alpha, uint32_t keep, int q, int c,
                                         int hA, const Magic& mk)
{
    constexpr int NG = 2;
    const int part = c & 1;

    // rescale the accumulators when a running maximum moved
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
        const float alA = __shfl(alpha, 2 * hA, 64), alB = __shfl(alpha, 2 * hA + 2, 64);
#pragma unroll
        for (int T = 0; T < 8; T++) {
            S.acc[T][0] *= alA;
            S.acc[T][1] *= alA;
            S.acc[T][2] *= alB;
            S.acc[T][3] *= alB;
        }
    }

    float sv[NG][16];
#pragma unroll
    for (int g = 0; g < NG; g++) read16f(lds + META_VS + g * 256 + 64 * q, sv[g]);
    uint32_t zv[2][4];
#pragma unroll
    for (int g = 0; g < 2; g++) read16b(lds + META_VZ + g * 64 + 16 * q, zv[g]);

#pragma unroll
    for (int u = 0; u < 2; u++) {
        if (!(keep & (1u << u))) continue;  // every V term of the 32 tokens skipped
        // A operand: p * s_v split into bf16 high part and bf16 remainder
        uint32_t pa[NG][4];
#pragma unroll
        for (int g = 0; g < NG; g++) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const int t = 2 * u + (j >> 2), r = j & 3;
                const int x = tok_of<VB>(t, r);
                const float pj = p[4 * t + r];
                float pp = pj * sv[g][x];
                if constexpr (PARTIAL) pp = pj > 0.0f ? pp : 0.0f;  // dead token: its scale bytes may be stale
                const float hi = __uint_as_float(__float_as_uint(pp) & 0xFFFF0000u);
                v[j] = part ? pp - hi : hi;
            }
#pragma unroll
            for (int k = 0; k < 4; k++) pa[g][k] = pack_bf16(v[2 * k], v[2 * k + 1]);
        }
        // correction operand: -(OFF + z) of each token, the same for every column
        uint32_t bz[2][4];
        neg_off_pairs<VB>(zv[0], u, bz[0]);
        neg_off_pairs<VB>(zv[1], u, bz[1]);
#pragma unroll
        for (int T = 0; T < 8; T++) {
            uint32_t bv[4];
            if constexpr (VB == 4) {
                const uint32_t w = R.vr[T][u];
                bv[0] = pair4<0>(w, mk);
                bv[1] = pair4<1>(w, mk);
                bv[2] = pair4<2>(w, mk);
                bv[3] = pair4<3>(w, mk);
            } else if (u == 0) {
                bv[0] = pair6<0>(R.vr[T], mk);
                bv[1] = pair6<12>(R.vr[T], mk);
                bv[2] = pair6<24>(R.vr[T], mk);
                bv[3] = pair6<36>(R.vr[T], mk);
            } else {
                bv[0] = pair6<48>(R.vr[T], mk);
                bv[1] = pair6<60>(R.vr[T], mk);
                bv[2] = pair6<72>(R.vr[T], mk);
                bv[3] = pair6<84>(R.vr[T], mk);
            }
            const int gT = T >> 2;
            // sum_t p'(t) (-(OFF + z(t))), then + sum_t p'(t) (OFF + c(t)): the
            // offset never accumulates beyond 32 tokens
            S.acc[T] = mfma_16x16x32(pa[gT], bz[gT], S.acc[T]);
            S.acc[T] = mfma_16x16x32(pa[gT], bv, S.acc[T]);
        }
    }
}

// ---- 4 query heads per KV head: two token sets per product
// With 4 heads the 16 QK columns would hold only 8 (head, group) pairs, and
// every lane would score 16 tokens of which half belong to idle columns.
// Instead the K dimension of each QK product carries two 16-token sets: lane
// groups q = 0, 1 hold set 0 and q = 2, 3 set 1, q & 1 selecting the channel
// group; a product then covers 32 tokens x 16 channels, the columns are
// (set s, head h, group g) = 8 s + 2 h + g, and each lane scores 8 tokens of
// a block.  In the P.V products the rows are (set, head, part): a set's rows
// take the A operand of that set's tokens and zero elsewhere, so the two
// sets' rows add up to the head's sum.  The token of K index j in lane group
// q is unchanged (16 q + 8 u + tok_of(2 u, j) for tile pair u), so the V
// operands are those of the 8-head layout.

// Token (0..63) of the lane's score (u, i): lane group q, token set s.
template <int VB>
__device__ __forceinline__ int set_tok(int q, int s, int u, int i)
{
    return 16 * q + tok_of<VB>(2 * u, i) + (VB == 4 ? 2 : 4) * s;
}

// fp32 values of the lane's 8 tokens from a 64-slot LDS section.
template <int VB>
__device__ __forceinline__ void set_floats(const uint8_t* sec, int q, int s, float (&v)[8])
{
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int t = set_tok<VB>(q, s, u, 0);
        if constexpr (VB == 4) {  // tokens t, t + 4, t + 1, t + 5
            const float2 a = *(const float2*)(sec + 4 * t), b = *(const float2*)(sec + 4 * (t + 4));
            v[4 * u] = a.x; v[4 * u + 1] = b.x; v[4 * u + 2] = a.y; v[4 * u + 3] = b.y;
        } else {  // tokens t .. t + 3
            const float4 a = *(const float4*)(sec + 4 * t);
            v[4 * u] = a.x; v[4 * u + 1] = a.y; v[4 * u + 2] = a.z; v[4 * u + 3] = a.w;
        }
    }
}

// Zero points (uint8) of the lane's 8 tokens from a 64-slot LDS section, as fp32.
template <int VB>
__device__ __forceinline__ void set_bytes(const uint8_t* sec, int q, int s, float (&v)[8])
{
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int t = set_tok<VB>(q, s, u, 0);
        if constexpr (VB == 4) {
            const uint32_t a = *(const uint16_t*)(sec + t), b = *(const uint16_t*)(sec + t + 4);
            v[4 * u] = (float)(a & 0xFFu); v[4 * u + 1] = (float)(b & 0xFFu);
            v[4 * u + 2] = (float)(a >> 8); v[4 * u + 3] = (float)(b >> 8);
        } else {
            const uint32_t a = *(const uint32_t*)(sec + t);
#pragma unroll
            for (int i = 0; i < 4; i++) v[4 * u + i] = (float)((a >> (8 * i)) & 0xFFu);
        }
    }
}

// K codes: for tile pair u, lane (q, c) holds channel group q & 1 (48
// contiguous bytes) of the token of QK row c in set q >> 1; words 0..11 go
// to kr[2u][0..5], kr[2u + 1][0..5].
template <int VB>
__device__ __forceinline__ void load_k_sets(BlockRegs<VB>& R, const uint8_t* ch, uint32_t off_kc, int c, int q)
{
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const uint32_t tok = 16 * (c >> 2) + set_tok<VB>(0, q >> 1, u, c & 3);
        const uint4* p = (const uint4*)(ch + (off_kc + tok * 96 + 48 * (q & 1)));
        const uint4 x0 = p[0], x1 = p[1], x2 = p[2];
        R.kr[2 * u][0] = x0.x; R.kr[2 * u][1] = x0.y; R.kr[2 * u][2] = x0.z;
        R.kr[2 * u][3] = x0.w; R.kr[2 * u][4] = x1.x; R.kr[2 * u][5] = x1.y;
        R.kr[2 * u + 1][0] = x1.z; R.kr[2 * u + 1][1] = x1.w; R.kr[2 * u + 1][2] = x2.x;
        R.kr[2 * u + 1][3] = x2.y; R.kr[2 * u + 1][4] = x2.z; R.kr[2 * u + 1][5] = x2.w;
    }
}

// Q.K of both tile pairs: 8 products each, product m taking pairs
// 4 (m & 1) .. 4 (m & 1) + 3 of the lane's 16-channel run m >> 1.
template <int VB>
__device__ __forceinline__ void block_qk_sets(const BlockRegs<VB>& R, const uint32_t (&qb)[8][4], float q128,
                                              const Magic& mk, f32x4_t (&dot)[2])
{
#pragma unroll
    for (int u = 0; u < 2; u++) {
        uint32_t pr[4][8];
        k16_pairs(R.kr[2 * u][0], R.kr[2 * u][1], R.kr[2 * u][2], mk, pr[0]);
        k16_pairs(R.kr[2 * u][3], R.kr[2 * u][4], R.kr[2 * u][5], mk, pr[1]);
        k16_pairs(R.kr[2 * u + 1][0], R.kr[2 * u + 1][1], R.kr[2 * u + 1][2], mk, pr[2]);
        k16_pairs(R.kr[2 * u + 1][3], R.kr[2 * u + 1][4], R.kr[2 * u + 1][5], mk, pr[3]);
        f32x4_t d4 = {-q128, -q128, -q128, -q128};  // removes the 128 offset of the codes
#pragma unroll
        for (int m = 0; m < 8; m++) {
            const uint32_t ka[4] = {pr[m >> 1][4 * (m & 1)], pr[m >> 1][4 * (m & 1) + 1],
                                    pr[m >> 1][4 * (m & 1) + 2], pr[m >> 1][4 * (m & 1) + 3]};
            d4 = mfma_16x16x32(ka, qb[m], d4);
        }
        dot[u] = d4;
    }
}

// block_softmax for the two-set layout: the lane's 8 scores are tokens
// set_tok(q, c >> 3, u, i) of head (c >> 1) & 3; the running (m, L) of a head
// is reduced over both sets, so every lane of a head holds the same values.
template <int VB, bool PARTIAL, bool KN>
__device__ __forceinline__ float block_softmax_sets(const f32x4_t (&dot)[2], const uint8_t* lds, SplitState& S,
                                                    float qsum, float score_scale, float tau_low, int nlive, int q,
                                                    int c, float (&p)[8], uint32_t& keep, float* srow,
                                                    uint32_t* mrow, int mcol)
{
    const int gc = c & 1, s = c >> 3;
    float sk[8], zk[8];
    set_floats<VB>(lds + gc * 256, q, s, sk);
    set_bytes<VB>(lds + META_KZ + gc * 64, q, s, zk);
    float rk[8];  // direction-preserving K: the norm factors of the lane's 8 tokens
    if constexpr (KN) set_floats<VB>(lds + META_BYTES, q, s, rk);
    float sc[8];
    float bmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; u++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int x = 4 * u + i;
            // the group share rounded before the exchange, as in block_softmax
            const float pg = mul_rounded(sk[x], dot[u][i] - zk[x] * qsum);
            float s2 = pg + xor1(pg);
            if constexpr (KN) s2 *= rk[x];
            if constexpr (PARTIAL) s2 = set_tok<VB>(q, s, u, i) < nlive ? s2 : -INFINITY;
            sc[x] = s2;
            bmax = fmaxf(bmax, s2);
        }
    }
    if (srow != nullptr && gc == 0) {
        float v[8];
#pragma unroll
        for (int x = 0; x < 8; x++) v[x] = sc[x] * score_scale;
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const int t = set_tok<VB>(q, s, u, 0);
            if constexpr (PARTIAL) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int ti = set_tok<VB>(q, s, u, i);
                    if (ti < nlive) srow[ti] = v[4 * u + i];
                }
            } else if constexpr (VB == 4) {
                *(float2*)(srow + t) = make_float2(v[4 * u], v[4 * u + 2]);
                *(float2*)(srow + t + 4) = make_float2(v[4 * u + 1], v[4 * u + 3]);
            } else {
                *(float4*)(srow + t) = make_float4(v[4 * u], v[4 * u + 1], v[4 * u + 2], v[4 * u + 3]);
            }
        }
    }
    bmax = rows_max(fmaxf(bmax, xor8(bmax))) * score_scale;  // both sets, base 2
    const float m_new = bmax > S.m_run + 8.0f ? bmax : S.m_run;
    const float m_ref = PARTIAL && m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(S.m_run - m_ref);
    float bsum = 0.0f;
#pragma unroll
    for (int x = 0; x < 8; x++) {
        p[x] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[x], score_scale, -m_ref));
        bsum += p[x];
    }
    S.l_run = S.l_run * alpha + rows_sum(bsum + xor8(bsum));
    S.m_run = m_new;
    keep = 3u;
    if (tau_low > 0.0f) {
        const float thr = tau_low * S.l_run;
        bool k0 = false, k1 = false;
#pragma unroll
        for (int x = 0; x < 8; x++) {
            p[x] = p[x] < thr ? 0.0f : p[x];
            if (x < 4) k0 |= p[x] > 0.0f;  // tile pair 0
            else k1 |= p[x] > 0.0f;
        }
        keep = (__builtin_amdgcn_ballot_w64(k0) ? 1u : 0u) | (__builtin_amdgcn_ballot_w64(k1) ? 2u : 0u);
        if (mrow != nullptr && gc == 0) {  // a live token's weight is 0 here exactly when it was below thr
#pragma unroll
            for (int u = 0; u < 2; u++) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int tok = set_tok<VB>(q, s, u, i);
                    if ((!PARTIAL || tok < nlive) && p[4 * u + i] == 0.0f) mark_skipped(mrow, mcol + tok);
                }
            }
        }
    }
    return alpha;
}

// block_pv for the two-set layout: row c = (set c >> 3, head, part c & 1);
// K indices 4 s .. 4 s + 3 of the lane's 8 carry its own tokens, the others
// zero.  Both V groups have an A operand of their own.
template <int VB, bool PARTIAL>
__device__ __forceinline__ void block_pv_sets(const BlockRegs<VB>& R, const uint8_t* lds, SplitState& S,
                                              const float (&p)[8], float alpha, uint32_t keep, int q, int c,
                                              int hA, const Magic& mk)
{
    const int part = c & 1, s = c >> 3;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
        const float alA = __shfl(alpha, 2 * hA, 64), alB = __shfl(alpha, 2 * hA + 2, 64);
#pragma unroll
        for (int T = 0; T < 8; T++) {
            S.acc[T][0] *= alA;
            S.acc[T][1] *= alA;
            S.acc[T][2] *= alB;
            S.acc[T][3] *= alB;
        }
    }
    float sv[2][8];
    set_floats<VB>(lds + META_VS, q, s, sv[0]);
    set_floats<VB>(lds + META_VS + 256, q, s, sv[1]);
    uint32_t zv[2][4];
#pragma unroll
    for (int g = 0; g < 2; g++) read16b(lds + META_VZ + g * 64 + 16 * q, zv[g]);

#pragma unroll
    for (int u = 0; u < 2; u++) {
        if (!(keep & (1u << u))) continue;
        uint32_t pa[2][4];
#pragma unroll
        for (int g = 0; g < 2; g++) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float pj = p[4 * u + i];
                float pp = pj * sv[g][4 * u + i];
                if constexpr (PARTIAL) pp = pj > 0.0f ? pp : 0.0f;  // dead token: its scale bytes may be stale
                const float hi = __uint_as_float(__float_as_uint(pp) & 0xFFFF0000u);
                v[i] = part ? pp - hi : hi;
            }
            const uint32_t d0 = pack_bf16(v[0], v[1]), d1 = pack_bf16(v[2], v[3]);
            pa[g][0] = s ? 0u : d0;
            pa[g][1] = s ? 0u : d1;
            pa[g][2] = s ? d0 : 0u;
            pa[g][3] = s ? d1 : 0u;
        }
        uint32_t bz[2][4];
        neg_off_pairs<VB>(zv[0], u, bz[0]);
        neg_off_pairs<VB>(zv[1], u, bz[1]);
#pragma unroll
        for (int T = 0; T < 8; T++) {
            uint32_t bv[4];
            if constexpr (VB == 4) {
                const uint32_t w = R.vr[T][u];
                bv[0] = pair4<0>(w, mk);
                bv[1] = pair4<1>(w, mk);
                bv[2] = pair4<2>(w, mk);
                bv[3] = pair4<3>(w, mk);
            } else if (u == 0) {
                bv[0] = pair6<0>(R.vr[T], mk);
                bv[1] = pair6<12>(R.vr[T], mk);
                bv[2] = pair6<24>(R.vr[T], mk);
                bv[3] = pair6<36>(R.vr[T], mk);
            } else {
                bv[0] = pair6<48>(R.vr[T], mk);
                bv[1] = pair6<60>(R.vr[T], mk);
                bv[2] = pair6<72>(R.vr[T], mk);
                bv[3] = pair6<84>(R.vr[T], mk);
            }
            const int gT = T >> 2;
            S.acc[T] = mfma_16x16x32(pa[gT], bz[gT], S.acc[T]);
            S.acc[T] = mfma_16x16x32(pa[gT], bv, S.acc[T]);
        }
    }
}

// ---- the decode step's own append (lkv_append_decode)
// The wave whose split holds a sequence's newest token (position len - 1,
// in the split's last block) quantises that token's K and V row with the
// append kernel's quantiser (the same codes, scales and zero points:
// group-wise asymmetric quantisation of the TurboQuant page, K6 and 4- or
// 6-bit V of the Super KV Compression page, first layer).  It writes the row
// into the pool for later steps and places it in its own registers for the
// block it reads, whose loads may precede those writes: nothing is read back,
// and no store is waited for.  Lane l holds channels 2l and 2l + 1 of the
// row, so a 64-channel group is 32 lanes.

// Channels 2 lane and 2 lane + 1 of row `row` of a [rows][128] input, as fp32.
__device__ __forceinline__ void load_pair(const void* p, int64_t row, int dt, int lane, float (&x)[2])
{
    if (dt == LKV_F32) {
        const float2 t = ((const float2*)p)[row * 64 + lane];
        x[0] = t.x;
        x[1] = t.y;
    } else {
        const uint32_t t = ((const uint32_t*)p)[row * 64 + lane];
        if (dt == LKV_BF16) {
            x[0] = __uint_as_float(t << 16);
            x[1] = __uint_as_float(t & 0xFFFF0000u);
        } else {
            x[0] = __half2float(__ushort_as_half((uint16_t)(t & 0xFFFFu)));
            x[1] = __half2float(__ushort_as_half((uint16_t)(t >> 16)));
        }
    }
}

// The quantised new row as the wave holds it.
struct NewRow {
    uint32_t kw;         // K row word 3 (lane >> 3) + (lane & 7) (lanes with lane & 7 < 3; 24 words)
    uint32_t vq;         // V codes of channels 2 lane (bits 0..7) and 2 lane + 1 (bits 8..15)
    float ks0, ks1, vs0, vs1;  // scales of groups 0 and 1 (uniform)
    int kz0, kz1, vz0, vz1;    // zero points (uniform)
};

template <int VB>
__device__ __forceinline__ void quantize_new_row(const float (&xk)[2], const float (&xv)[2], int lane, NewRow& r)
{
    QRow<2> k, v;
    quantize_fast<2, 64>(xk, 6, k);
    quantize_fast<2, 64>(xv, VB, v);
    if (k.slow) quantize_exact<2>(xk, 6, k);
    if (v.slow) quantize_exact<2>(xv, VB, v);
    // K: the lane's two codes are 12 bits at bit 12 lane of the 96-byte row;
    // 8 lanes fill 3 words, held by the first three of them
    const uint32_t k12 = (uint32_t)k.q[0] | ((uint32_t)k.q[1] << 6);
    const int m = lane >> 3, j = lane & 7;
    uint32_t vals[8], w[3];
#pragma unroll
    for (int i = 0; i < 8; i++) vals[i] = (uint32_t)__shfl((int)k12, 8 * m + i, 64);
    pack_values<12, 8, 3>(vals, w);
    r.kw = j == 0 ? w[0] : (j == 1 ? w[1] : w[2]);
    r.vq = (uint32_t)v.q[0] | ((uint32_t)v.q[1] << 8);
    auto from = [](float x, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l)); };
    r.ks0 = from(k.s, 0);
    r.ks1 = from(k.s, 32);
    r.vs0 = from(v.s, 0);
    r.vs1 = from(v.s, 32);
    r.kz0 = __builtin_amdgcn_readlane(k.z, 0);
    r.kz1 = __builtin_amdgcn_readlane(k.z, 32);
    r.vz0 = __builtin_amdgcn_readlane(v.z, 0);
    r.vz1 = __builtin_amdgcn_readlane(v.z, 32);
}

// The K codes, scales and zero points of the new row into slot `slot` of
// chunk ch (the V codes are written by patch_v, merged with the words'
// other slots).
__device__ __forceinline__ void store_new_row(const NewRow& r, uint8_t* ch, const Fmt& f, int slot, int lane)
{
    if ((lane & 7) < 3) ((uint32_t*)(ch + f.off_kc + slot * 96))[3 * (lane >> 3) + (lane & 7)] = r.kw;
    if (lane < 2) {  // lane g: group g
        ((float*)(ch + f.off_ks))[lane * BT + slot] = lane ? r.ks1 : r.ks0;
        ((float*)(ch + f.off_vs))[lane * BT + slot] = lane ? r.vs1 : r.vs0;
        ch[f.off_kz + lane * BT + slot] = (uint8_t)(lane ? r.kz1 : r.kz0);
        ch[f.off_vz + lane * BT + slot] = (uint8_t)(lane ? r.vz1 : r.vz0);
    }
}

// The new row's scales and zero points into the block's staged metadata.
__device__ __forceinline__ void patch_meta(const NewRow& r, uint8_t* lds, int slot, int lane)
{
    if (lane < 2) {
        *(float*)(lds + lane * 256 + 4 * slot) = lane ? r.ks1 : r.ks0;
        *(float*)(lds + META_VS + lane * 256 + 4 * slot) = lane ? r.vs1 : r.vs0;
        lds[META_KZ + lane * 64 + slot] = (uint8_t)(lane ? r.kz1 : r.kz0);
        lds[META_VZ + lane * 64 + slot] = (uint8_t)(lane ? r.vz1 : r.vz0);
    }
}

// K row word w of the new row, from the lane that holds it.
__device__ __forceinline__ uint32_t new_k_word(const NewRow& r, int w)
{
    return (uint32_t)__shfl((int)r.kw, 8 * (w / 3) + w % 3, 64);
}

// The new row's K codes into the block's K registers: the lanes whose
// tiles hold token `slot` (load_k_sets / load_k layouts).
template <int VB, bool SETS>
__device__ __forceinline__ void patch_k(BlockRegs<VB>& R, const NewRow& r, int slot, int q, int c)
{
    if constexpr (SETS) {
        uint32_t w[12];
#pragma unroll
        for (int i = 0; i < 12; i++) w[i] = new_k_word(r, 12 * (q & 1) + i);
#pragma unroll
        for (int u = 0; u < 2; u++) {
            const bool hit = 16 * (c >> 2) + set_tok<VB>(0, q >> 1, u, c & 3) == slot;
#pragma unroll
            for (int i = 0; i < 6; i++) {
                R.kr[2 * u][i] = hit ? w[i] : R.kr[2 * u][i];
                R.kr[2 * u + 1][i] = hit ? w[6 + i] : R.kr[2 * u + 1][i];
            }
        }
    } else {
        uint32_t w[6];
#pragma unroll
        for (int i = 0; i < 6; i++) w[i] = new_k_word(r, 6 * q + i);
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const bool hit = 16 * (c >> 2) + tok_of<VB>(t, c & 3) == slot;
#pragma unroll
            for (int i = 0; i < 6; i++) R.kr[t][i] = hit ? w[i] : R.kr[t][i];
        }
    }
}

// The new row's V codes into the block's V registers (lane group q holds
// tokens 16 q .. 16 q + 15 of channels 16 T + c), and the merged words, the
// pool's new contents, into chunk ch.
template <int VB>
__device__ __forceinline__ void patch_v(BlockRegs<VB>& R, const NewRow& r, int slot, int q, int c, uint8_t* ch,
                                        uint32_t off_vc)
{
    constexpr int NW = VB == 4 ? 2 : 3;
    const int bit = VB * (slot & 15), wi = bit >> 5, sh = bit & 31;
    const bool spill = sh + VB > 32;  // a 6-bit field across two words
    const uint32_t fm = (1u << VB) - 1u;
    const bool mine = q == (slot >> 4);
#pragma unroll
    for (int T = 0; T < 8; T++) {
        const uint32_t x = (uint32_t)__shfl((int)r.vq, 8 * T + (c >> 1), 64);
        const uint32_t code = (c & 1) ? (x >> 8) & 0xFFu : x & 0xFFu;
        uint32_t* row = (uint32_t*)(ch + off_vc + (16 * T + c) * (8 * VB)) + (VB * q) / 2;
#pragma unroll
        for (int w = 0; w < NW; w++) {
            uint32_t m = 0u, v = 0u;
            if (w == wi) {
                m = fm << sh;
                v = code << sh;
            } else if (w == wi + 1 && spill) {
                m = fm >> (32 - sh);
                v = code >> (32 - sh);
            }
            if (mine && m != 0u) {
                R.vr[T][w] = (R.vr[T][w] & ~m) | v;
                row[w] = R.vr[T][w];
            }
        }
    }
}

// One wave's split: split sp of KV head blockIdx.y of grid entry blockIdx.z.
// PAIR (the 8-head layout over 4 query heads per KV head): grid entry
// blockIdx.z is a pair of consecutive query tokens (2i, 2i + 1) of one
// sequence of a multi-token call; the layout's heads 0-3 are token 2i's
// four heads and heads 4-7 token 2i + 1's, so every block is unpacked once
// for both.  The earlier token's causal prefix is one token shorter: its
// columns are masked in the split's last blocks.  An odd T's last token is
// paired with itself and its second copy is not written.
//
// LO: the partial goes to lo (LDS, [G][D + 2]) instead of the workspace, for
// a workgroup that merges its waves' splits before anything leaves the CU.
template <int VB, int G, bool KN, bool PAIR = false, bool DBG = false, bool APP = false, bool LO = false>
__device__ __forceinline__ void split_body(const MfmaArgs& a, const int sp, const int kvh, const int b, const int lane,
                                           uint4* meta_lds, float* lo = nullptr)
{
    static_assert(G == 4 || G == 8, "4 or 8 query heads per KV head");
    static_assert(!PAIR || G == 8, "a pair fills the 8-head layout");
    constexpr bool SETS = G == 4;  // the two-set layout
    constexpr int D = 128;
    const SegArgs& sg = a.seg;
    const Fmt& f = sg.f;
    const int c = lane & 15, q = lane >> 4;
    const int t0 = sp * a.split_tokens;
    // the split's block-table entries (at most 64, one per lane) do not
    // depend on the length: they are requested together with it
    // (the sequence and length are uniform: computed before the lane-dependent
    // load, so that they stay in scalar registers)
    int seq, len, e0 = b, e1 = b, len0 = 0;  // PAIR: the tokens' entries and the earlier one's length
    if constexpr (PAIR) {
        const int T = sg.q_per_seq, np = (T + 1) >> 1;
        const int tk = 2 * (b % np);
        e0 = b / np * T + tk;
        e1 = tk + 1 < T ? e0 + 1 : e0;
        seq = entry_seq(sg, e0);
        len0 = max(0, min(entry_len(sg, e0), sg.len_cap));
        len = max(0, min(entry_len(sg, e1), sg.len_cap));
    } else {
        seq = entry_seq(sg, b);
        len = max(0, min(entry_len(sg, b), sg.len_cap));
    }
    // partial row (entry, query head) of layout head hh, and whether it is written
    auto prow = [&](int hh) -> int64_t {
        if constexpr (PAIR) return (int64_t)(hh >= 4 ? e1 : e0) * a.num_q_heads + kvh * 4 + (hh & 3);
        else return (int64_t)b * a.num_q_heads + kvh * G + hh;
    };
    auto pwrite = [&](int hh) { return !PAIR || hh < 4 || e1 != e0; };
    const int32_t* bt = sg.block_table + (int64_t)seq * sg.max_blocks + t0 / BT;
    const int bt_lane = lane < min(64, sg.max_blocks - t0 / BT) ? bt[lane] : 0;
    asm volatile("" ::: "memory");  // both loads are issued before either is waited for
    const int t1 = min(t0 + a.split_tokens, len);
    if (t1 <= t0) {  // a split past the end: only (m, L) = (-inf, 0), its o row is never read
        if constexpr (PAIR) {
            if (lane < G && pwrite(lane)) {
                float* p = a.partials + (prow(lane) * a.total_splits + sg.split_base + sp) * (D + 2);
                p[D] = -INFINITY;
                p[D + 1] = 0.0f;
            }
        } else if (LO && lane < G) {
            lo[lane * (D + 2) + D] = -INFINITY;
            lo[lane * (D + 2) + D + 1] = 0.0f;
        } else if (lane < G) {
            float* p = a.partials + (((int64_t)b * a.num_q_heads + kvh * G + lane) * a.total_splits +
                                     sg.split_base + sp) * (D + 2);
            p[D] = -INFINITY;
            p[D + 1] = 0.0f;
        }
        return;
    }

    // ---- roles of this lane
    // 8-head layout: QK column c -> (head hc, group gc), P.V row c -> (head
    // hc, part c & 1).  Two-set layout: QK column c -> (set c >> 3, head hc,
    // group gc), P.V row c -> (set c >> 3, head hc, part c & 1).
    const int hc = G == 8 ? (c >> 1) : ((c >> 1) & 3);
    const int gc = c & 1;
    const int part = c & 1;
    const int head = kvh * G + hc;
    // heads of the P.V output rows held by this lane (rows 4q .. 4q+3)
    const int hA = G == 8 ? 2 * q : 2 * (q & 1);
    // this lane's head's score row, at the split's first token
    const int64_t srow0 = ((int64_t)b * a.num_q_heads + head) * sg.score_stride + sg.tok_base + t0;
    // this lane's head's skip-mask row (test entry point only)
    uint32_t* const mrow = DBG && sg.skip_mask != nullptr && pwrite(hc)
                               ? sg.skip_mask + (PAIR ? prow(hc) : (int64_t)b * a.num_q_heads + head) * sg.mask_stride
                               : nullptr;

    // ---- Q as the QK B operand.  8-head layout: this lane group (q) holds
    // channels [32q, 32q + 32), in group q >> 1; zero unless that is the
    // column's group.  Two-set layout: lane group q holds all 64 channels of
    // group q & 1 for set q >> 1; zero unless both are the column's.  Q is
    // loaded before the first block's loads are issued and turned into the
    // operand while that block is in flight.  (Every lane loads: the lanes of
    // one column read the same bytes, so the idle ones add no lines.)
    constexpr int NQ = SETS ? 8 : 4;  // 16-byte pieces per lane
    const bool qlive = SETS ? q == 2 * (c >> 3) + gc : (q >> 1) == gc;
    uint4 qraw[NQ];
    {
        const int64_t qrow = PAIR ? prow(hc) : (int64_t)b * a.num_q_heads + head;
        const uint4* src = (const uint4*)(a.q + qrow * D + (SETS ? 64 * gc : 32 * q));
#pragma unroll
        for (int i = 0; i < NQ; i++) qraw[i] = src[i];
    }
    const int nblk = (t1 - t0 + BT - 1) / BT;
    // APP: this wave appends the newest token (position len - 1, in its last
    // block) when the token falls in its split; the row's inputs are
    // requested together with Q
    const bool app = APP && (len - 1) / a.split_tokens == sp;
    float xk[2] = {0.0f, 0.0f}, xv[2] = {0.0f, 0.0f};
    if constexpr (APP) {
        if (app) {
            load_pair(a.k_new, (int64_t)seq * f.H + kvh, a.kv_dtype, lane, xk);
            load_pair(a.v_new, (int64_t)seq * f.H + kvh, a.kv_dtype, lane, xv);
        }
    }
    asm volatile("" ::: "memory");

    const uint8_t* lds = (const uint8_t*)meta_lds;

    // the split's block-table entries (at most 64), one per lane, so that
    // every chunk address is a register read instead of a memory round trip
    // end of this lane's column's tokens in the split, and of the tokens
    // every column has (they differ only for a pair: t1 belongs to the later
    // token, the earlier one ends a token sooner)
    const int tl0 = PAIR ? max(t0, min(t0 + a.split_tokens, len0)) : t1;
    const int tl = PAIR && c < 8 ? tl0 : t1;
    // format fields as plain values (kept in scalar registers)
    const uint8_t* const pool = sg.pool;
    const int64_t chunk = f.chunk;
    const int H = f.H;
    const uint32_t off_kc = (uint32_t)f.off_kc, off_vc = (uint32_t)f.off_vc, off_ks = (uint32_t)f.off_ks;
    auto chunk_of = [=](int k) {
        const int blk = __builtin_amdgcn_readlane(bt_lane, k);
        return pool + ((int64_t)blk * H + kvh) * chunk;
    };

    // Blocks in order.  The next block's metadata, K codes and V codes are
    // loaded as soon as this block no longer needs the registers they go to,
    // so they stream in while this block computes.  The last block loads
    // nothing more: a repeat of its non-temporal loads would come from HBM.
    BlockRegs<VB> R;
    {
        // the same issue order as inside the loop: metadata, K, V
        const uint8_t* c0 = chunk_of(0);
        load_meta<VB, KN>(R, c0, off_ks, lane);
        asm volatile("" ::: "memory");
        if constexpr (SETS) load_k_sets<VB>(R, c0, off_kc, c, q);
        else load_k<VB>(R, c0, off_kc, c, q);
        asm volatile("" ::: "memory");
        load_v<VB>(R, c0, off_vc, c, q);
        asm volatile("" ::: "memory");
    }
    // Q is used from here on (not earlier: the first block's loads go first)
#pragma unroll
    for (int i = 0; i < NQ; i++) asm volatile("" : "+v"(qraw[i].x), "+v"(qraw[i].y), "+v"(qraw[i].z), "+v"(qraw[i].w));

    uint32_t qb[SETS ? 8 : 4][4];
    float qpart = 0.0f;
    {
        uint32_t qw[4 * NQ];  // channels 2i, 2i+1 of the lane's run
#pragma unroll
        for (int i = 0; i < NQ; i++) {
            qw[4 * i] = qlive ? qraw[i].x : 0u;
            qw[4 * i + 1] = qlive ? qraw[i].y : 0u;
            qw[4 * i + 2] = qlive ? qraw[i].z : 0u;
            qw[4 * i + 3] = qlive ? qraw[i].w : 0u;
        }
#pragma unroll
        for (int i = 0; i < 4 * NQ; i++) qpart += __uint_as_float(qw[i] << 16) + __uint_as_float(qw[i] & 0xFFFF0000u);
        // product m (two-set layout) or K-step m (8-head layout): pairs
        // 4(m&1) .. 4(m&1)+3 of the 16-channel run m>>1, the pairing the K
        // codes use; bytes of channel ca (low half) and cb (high half)
#pragma unroll
        for (int m = 0; m < (SETS ? 8 : 4); m++) {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int pj = 4 * (m & 1) + j;
                const int ca = 16 * (m >> 1) + kpair_ch(pj, 0), cb = 16 * (m >> 1) + kpair_ch(pj, 1);
                const uint32_t sel = ((ca & 1) ? 0x0302u : 0x0100u) | (((cb & 1) ? 0x0706u : 0x0504u) << 16);
                qb[m][j] = __builtin_amdgcn_perm(qw[cb >> 1], qw[ca >> 1], sel);
            }
        }
    }
    const float qsum = rows_sum(qpart);
    const float q128 = 128.0f * qsum;
    // APP: quantise the new row while the first block is in flight (its
    // inputs are not waited for before the block's loads are issued), and
    // write its K codes and metadata for later steps
    NewRow nr{};
    const int app_slot = (len - 1) & (BT - 1);
    if constexpr (APP) {
        asm volatile("" : "+v"(xk[0]), "+v"(xk[1]), "+v"(xv[0]), "+v"(xv[1]));
        if (app) {
            quantize_new_row<VB>(xk, xv, lane, nr);
            store_new_row(nr, (uint8_t*)chunk_of(nblk - 1), f, app_slot, lane);
        }
    }

    const Magic mk = make_magic();
    SplitState S;
    S.m_run = -INFINITY;
    S.l_run = 0.0f;
#pragma unroll
    for (int T = 0; T < 8; T++) S.acc[T] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // (the empty asm statements keep the compiler from moving the loads to
    // their first use)
    auto block = [&](int k, auto partial, auto prefetch) {
        constexpr bool PARTIAL = decltype(partial)::value;
        constexpr bool MORE = decltype(prefetch)::value;  // load block k + 1 (false: the split's last block)
        const uint8_t* cn = MORE ? chunk_of(k + 1) : nullptr;
        // raised wave priority from the block's start until the next block's
        // K loads are issued: a wave whose data has arrived gets to its next
        // loads ahead of the other wave's softmax and P.V
        __builtin_amdgcn_s_setprio(1);
        stage_meta<KN>(R.meta, meta_lds, lane);
        if constexpr (APP && !MORE) {
            // the split's last block holds the appended token
            if (app) {
                patch_meta(nr, (uint8_t*)meta_lds, app_slot, lane);
                patch_k<VB, SETS>(R, nr, app_slot, q, c);
            }
        }
        if constexpr (MORE) load_meta<VB, KN>(R, cn, off_ks, lane);
        asm volatile("" ::: "memory");
        f32x4_t dot[SETS ? 2 : 4];
        if constexpr (SETS) block_qk_sets<VB>(R, qb, q128, mk, dot);
        else block_qk<VB>(R, qb, q128, mk, dot);
        if constexpr (MORE) {
            if constexpr (SETS) load_k_sets<VB>(R, cn, off_kc, c, q);
            else load_k<VB>(R, cn, off_kc, c, q);
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_setprio(0);
        const int nlive = min(BT, tl - t0 - k * BT);  // PAIR: this lane's column's (may be <= 0)
        float p[SETS ? 8 : 16];
        uint32_t keep;
        float* srow = !PAIR && sg.scores != nullptr ? sg.scores + srow0 + (int64_t)k * BT : nullptr;
        const int mcol = sg.tok_base + t0 + k * BT;
        if constexpr (SETS) {
            const float alpha = block_softmax_sets<VB, PARTIAL, KN>(dot, lds, S, qsum, a.score_scale, a.tau_low,
                                                                    nlive, q, c, p, keep, srow, mrow, mcol);
            if constexpr (APP && !MORE) {
                if (app) patch_v<VB>(R, nr, app_slot, q, c, (uint8_t*)chunk_of(k), off_vc);
            }
            block_pv_sets<VB, PARTIAL>(R, lds, S, p, alpha, keep, q, c, hA, mk);
        } else {
            const float alpha = block_softmax<VB, PARTIAL, KN>(dot, lds, S, qsum, a.score_scale, a.tau_low, nlive, q,
                                                               c, p, keep, srow, mrow, mcol);
            if constexpr (APP && !MORE) {
                if (app) patch_v<VB>(R, nr, app_slot, q, c, (uint8_t*)chunk_of(k), off_vc);
            }
            block_pv<VB, PARTIAL>(R, lds, S, p, alpha, keep, q, c, hA, mk);
        }
        if constexpr (MORE) load_v<VB>(R, cn, off_vc, c, q);
        asm volatile("" ::: "memory");
    };
    // full blocks, then the split's last block if it has dead slots (PAIR:
    // blocks full for both tokens, then the rest, at most two, masked per
    // column).  The last block is an instance of its own that loads nothing
    // more.
    const int nfull = (tl0 - t0) / BT;
    int k = 0;
    for (; k < min(nfull, nblk - 1); k++) block(k, std::false_type{}, std::true_type{});
    if constexpr (PAIR) {
        for (; k < nblk - 1; k++) block(k, std::true_type{}, std::true_type{});
    }
    if (k < nfull) block(k, std::false_type{}, std::false_type{});
    else block(k, std::true_type{}, std::false_type{});

    // ---- write the partial (o, m, L) of every head of the group
    // P.V output: lane (column c, row group q) holds rows 4q .. 4q+3 of each
    // channel tile T; rows 4q, 4q+1 are head hA (hi, lo), 4q+2, 4q+3 head hA+1
    // (two-set layout: of token set q >> 1).
    if constexpr (PAIR) {
        // rows hA, hA + 1 belong to one token (hA even)
        const int64_t soff = (int64_t)(sg.split_base + sp) * (D + 2);
        float* pa = a.partials + prow(hA) * a.total_splits * (D + 2) + soff;
        float* pb = a.partials + prow(hA + 1) * a.total_splits * (D + 2) + soff;
        if (pwrite(hA)) {
#pragma unroll
            for (int T = 0; T < 8; T++) {
                pa[16 * T + c] = S.acc[T][0] + S.acc[T][1];
                pb[16 * T + c] = S.acc[T][2] + S.acc[T][3];
            }
        }
        if (q == 0 && part == 0 && pwrite(hc)) {
            float* pm = a.partials + prow(hc) * a.total_splits * (D + 2) + soff;
            pm[D] = S.m_run;
            pm[D + 1] = S.l_run;
        }
        return;
    }
    float* base = a.partials + ((int64_t)b * a.num_q_heads + kvh * G) * a.total_splits * (D + 2);
    const int64_t hstride = (int64_t)a.total_splits * (D + 2);
    const int64_t soff = (int64_t)(sg.split_base + sp) * (D + 2);
#pragma unroll
    for (int T = 0; T < 8; T++) {
        float o0 = S.acc[T][0] + S.acc[T][1], o1 = S.acc[T][2] + S.acc[T][3];
        if constexpr (SETS) {
            // rows of set 1 (lane groups 2, 3) add to those of set 0; the
            // lane groups of V group T >> 2 write the sum
            o0 = halves_sum(o0);
            o1 = halves_sum(o1);
            if ((q >> 1) != (T >> 2)) continue;
        }
        if constexpr (LO) {
            lo[hA * (D + 2) + 16 * T + c] = o0;
            lo[(hA + 1) * (D + 2) + 16 * T + c] = o1;
        } else {
            base[hA * hstride + soff + 16 * T + c] = o0;
            base[(hA + 1) * hstride + soff + 16 * T + c] = o1;
        }
    }
    if (q == 0 && part == 0 && (G == 8 || c < 8)) {  // two-set layout: set 0's lane of the head
        if constexpr (LO) {
            lo[hc * (D + 2) + D] = S.m_run;
            lo[hc * (D + 2) + D + 1] = S.l_run;
        } else {
            base[hc * hstride + soff + D] = S.m_run;
            base[hc * hstride + soff + D + 1] = S.l_run;
        }
    }
}

// DBG: the same kernel that also records its skip decisions (the test entry
// point's skip mask); production launches take DBG = false, where the mask
// code is compiled out.
template <int VB, int G, bool KN, bool DBG>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void split_mfma_kernel(MfmaArgs a)
{
    __shared__ uint4 meta_lds[meta_bytes<KN>() / 16];
    split_body<VB, G, KN, false, DBG>(a, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x, meta_lds);
}

// Multi-token calls with 8 query heads per KV head: the T query tokens of
// one (split, KV head, sequence) item run in workgroups 8 apart, which the
// dispatcher sends to the same XCD one after another, so that the later
// tokens find the split's chunks in that XCD's L2 rather than read them
// from memory again.  1-D grid: ceil(items / 8) * 8 * T workgroups.
template <int VB, bool KN, bool DBG>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void split_mfma_multi8_kernel(MfmaArgs a)
{
    __shared__ uint4 meta_lds[meta_bytes<KN>() / 16];
    const int T = a.seg.q_per_seq, ns = a.seg.n_splits, H = a.seg.f.H;
    const int j = blockIdx.x / 8;
    const int t = j % T, item = j / T * 8 + blockIdx.x % 8;
    if (item >= a.items) return;
    split_body<VB, 8, KN, false, DBG>(a, item % ns, item / ns % H, item / ns / H * T + t, threadIdx.x, meta_lds);
}

// Query-token pairs of a multi-token call with 4 query heads per KV head
// (split_body's PAIR): grid z = sequence x ceil(T / 2) pairs.
template <int VB, bool KN, bool DBG>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void split_mfma_pair_kernel(MfmaArgs a)
{
    __shared__ uint4 meta_lds[meta_bytes<KN>() / 16];
    split_body<VB, 8, KN, true, DBG>(a, blockIdx.x, blockIdx.y, blockIdx.z, threadIdx.x, meta_lds);
}

// Both segments of a tiered cache in one launch: workgroups [0, n0) run the
// HIGH (V6) segment's splits, the rest the MID (V4) segment's, so the two
// share the machine instead of running one after the other.
template <int G, bool DBG>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void split_mfma_tiered_kernel(MfmaArgs a0,
                                                                                                       MfmaArgs a1)
{
    __shared__ uint4 meta_lds[META_BYTES / 16];
    const int sp = blockIdx.x;
    if (sp < a0.seg.n_splits) split_body<6, G, false, false, DBG>(a0, sp, blockIdx.y, blockIdx.z, threadIdx.x, meta_lds);
    else split_body<4, G, false, false, DBG>(a1, sp - a0.seg.n_splits, blockIdx.y, blockIdx.z, threadIdx.x, meta_lds);
}

// Decode with the step's own append (lkv_append_decode): the split holding
// each sequence's newest token writes that token's K and V row first.
//
// Dispatch order.  Workgroups start in linear order, one wave per SIMD
// first; on every SIMD the wave that started first finishes well ahead of
// the one that started second (about 15 us in a 60 us call), so the second
// half of the grid sets the call's time.  The splits holding a sequence's
// newest token, which carry the append, are therefore started first: the
// first half of the grid takes the last ceil(n/2) splits of every row (KV
// head, entry), newest first, the second half the rest.  Inside each half
// the split index runs fastest, so consecutive workgroups (which go to the
// XCDs in turn) still take different splits of one row.
//
// Compact order (a.compact entries, at most 64: a ragged batch).  Workgroup
// i takes the i-th (entry, KV head, split) that holds tokens, entries in
// turn, an entry's KV heads in turn, splits fastest; an empty sequence
// counts one split, which writes its (m, L) = (-inf, 0).  Every wave finds
// its item from the entries' lengths (a prefix sum over the lanes), so no
// slot goes to a split past a sequence's end and the items are spread over
// the XCDs evenly; workgroups past the last item return at once.  The wave
// with an entry's newest split also writes (-inf, 0) for the row's splits
// that have no workgroup, so the partials are complete for any merge.
__device__ __forceinline__ bool compact_item(const MfmaArgs& a, int lin, int& sp, int& row, int& nsp)
{
    const SegArgs& sg = a.seg;
    const int lane = threadIdx.x & 63, H = sg.f.H, st = a.split_tokens;
    int c = 0;
    if (lane < a.compact) c = max(1, min(sg.n_splits, (max(0, min(sg.seq_lens[lane], sg.len_cap)) + st - 1) / st));
    int x = H * c;  // inclusive prefix sum of the entries' items
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    const uint64_t past = __ballot(x > lin);
    if (past == 0) return false;
    const int e = __builtin_ctzll(past);
    const int ce = __builtin_amdgcn_readlane(c, e);
    const int k = lin - (__builtin_amdgcn_readlane(x, e) - H * ce);
    row = e * H + k / ce;
    sp = k % ce;
    nsp = ce;
    return true;
}

template <int VB, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void split_append_kernel(MfmaArgs a)
{
    __shared__ uint4 meta_lds[META_BYTES / 16];
    const int ns = a.seg.n_splits, H = a.seg.f.H;
    int sp, row, nsp = 0;
    if (a.compact > 0) {
        if (!compact_item(a, blockIdx.x, sp, row, nsp)) return;
    } else {
        const int P = (ns + 1) / 2;  // splits per row in the first half
        const int rows = (int)gridDim.x / ns;  // (KV head, entry) rows
        int lin = blockIdx.x, rev;
        if (lin < P * rows) {
            rev = lin % P;
            row = lin / P;
        } else {
            lin -= P * rows;
            rev = P + lin % (ns - P);
            row = lin / (ns - P);
        }
        sp = ns - 1 - rev;
    }
    split_body<VB, G, false, false, false, true>(a, sp, row % H, row / H, threadIdx.x, meta_lds);
    if (nsp > 0 && sp == nsp - 1) {  // the row's splits without a workgroup: (m, L) = (-inf, 0)
        const int b = row / H, kvh = row % H;
        for (int i = threadIdx.x; i < (ns - nsp) * G; i += 64) {
            float* p = a.partials + (((int64_t)b * a.num_q_heads + kvh * G + i % G) * a.total_splits +
                                     a.seg.split_base + nsp + i / G) * (128 + 2);
            p[128] = -INFINITY;
            p[129] = 0.0f;
        }
    }
}

// The decode step in one launch (lkv_append_decode_merged): the split kernel
// with the step's append also merges the splits.  A workgroup of MW = G
// waves (as many as query heads per KV head) takes MW consecutive splits of
// one (KV head, entry) row, one per wave, and
// each wave leaves its partial in LDS.  The workgroup merges those into one
// partial (wave w: head w), writes it through to the workspace
// as the row's partial j (device-scope stores, which reach the level every
// compute unit reads: the row's other workgroups run on other L2 caches),
// waits for the stores and counts itself in the row's counter (atomicInc,
// wrapping to 0 at the row's workgroup count nw).  The workgroup that counts
// last reads the row's nw partials back with device-scope loads and merges
// them into the output.  Only nw partials per head leave a compute unit, and
// the last workgroup's waves merge the heads side by side, one head each.
//
// Dispatch order as in split_append_kernel, by workgroup: the first half of
// the grid takes the last ceil(nw / 2) workgroups of every row (which hold
// the newest splits and the append), newest first, the second half the rest.
constexpr int MERGED_MAX_PARTIALS = 256;  // workgroup partials per row the last workgroup merges

//
// TIER: a tiered cache's two segments, HIGH (a, K6V6, which takes the new
// rows) and MID (a1, K6V4): a row's splits are HIGH's then MID's, so a
// workgroup may hold splits of both.
template <int VB, int G, bool TIER>
__global__ __launch_bounds__(64 * G) __attribute__((amdgpu_waves_per_eu(2))) void split_append_merged_kernel(
    MfmaArgs a, MfmaArgs a1)
{
    constexpr int D = 128, MW = G;
    __shared__ uint4 meta_lds[MW][META_BYTES / 16];
    __shared__ float part[MW][G][D + 2];
    __shared__ uint32_t ticket;
    // the wave index is uniform: read it into a scalar register, so that the
    // split and everything addressed from it stay scalar in split_body
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int ns0 = a.seg.n_splits, ns = ns0 + (TIER ? a1.seg.n_splits : 0), H = a.seg.f.H;
    const int nw = (ns + MW - 1) / MW;  // workgroups (merged partials) per row
    const int P = (nw + 1) / 2;         // workgroups per row in the first half
    const int rows = (int)gridDim.x / nw;
    int lin = blockIdx.x, rev, row;
    if (lin < P * rows) {
        rev = lin % P;
        row = lin / P;
    } else {
        lin -= P * rows;
        rev = P + lin % (nw - P);
        row = lin / (nw - P);
    }
    const int j = nw - 1 - rev;
    const int sp = j * MW + w, b = row / H, kvh = row % H;
    if (sp < ns0) {
        split_body<VB, G, false, false, false, true, true>(a, sp, kvh, b, lane, meta_lds[w], &part[w][0][0]);
    } else if (TIER && sp < ns) {
        split_body<4, G, false, false, false, false, true>(a1, sp - ns0, kvh, b, lane, meta_lds[w], &part[w][0][0]);
    } else if (lane < G) {  // past the row's last split: no token
        part[w][lane][D] = -INFINITY;
        part[w][lane][D + 1] = 0.0f;
    }
    __syncthreads();
    float* const prow0 = a.partials + ((int64_t)b * a.num_q_heads + kvh * G) * a.total_splits * (D + 2);
    {
        const int h = w;
        float2 ov[MW];
#pragma unroll
        for (int i = 0; i < MW; i++) ov[i] = *(const float2*)&part[i][h][2 * lane];
        const float mi = lane < MW ? part[lane][h][D] : -INFINITY;
        const float li = lane < MW ? part[lane][h][D + 1] : 0.0f;
        float M, L;
        const float2 o = merge128_partial(ov, mi, li, &M, &L);
        float* p = prow0 + ((int64_t)h * a.total_splits + j) * (D + 2);
        const uint64_t ob = (uint64_t)__float_as_uint(o.x) | ((uint64_t)__float_as_uint(o.y) << 32);
        __hip_atomic_store((uint64_t*)(p + 2 * lane), ob, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) {
            const uint64_t ml = (uint64_t)__float_as_uint(M) | ((uint64_t)__float_as_uint(L) << 32);
            __hip_atomic_store((uint64_t*)(p + D), ml, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are complete
    __syncthreads();                                  // ... and every wave's
    if (threadIdx.x == 0) ticket = atomicInc(a.counters + row, (unsigned)(nw - 1));
    __syncthreads();
    if (ticket != (uint32_t)(nw - 1)) return;
    // the row's last workgroup: wave w merges head w over the nw partials
    auto merge_row = [&](auto ch) __attribute__((always_inline)) {
        constexpr int CH = decltype(ch)::value;
        {
            const int h = w;
            const float* p = prow0 + (int64_t)h * a.total_splits * (D + 2);
            float2 ov[CH];
#pragma unroll
            for (int i = 0; i < CH; i++) {  // past the count: a counted row again, at weight 0
                const uint64_t v = __hip_atomic_load((const uint64_t*)(p + (int64_t)min(i, nw - 1) * (D + 2) + 2 * lane),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ov[i] = float2{__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32))};
            }
            uint64_t ml = 0xFF800000ull;  // (m, L) = (-inf, 0) past the count
            if (lane < nw)
                ml = __hip_atomic_load((const uint64_t*)(p + (int64_t)lane * (D + 2) + D), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            float M, inv;
            *(float2*)(a.out + ((int64_t)b * a.num_q_heads + kvh * G + h) * D + 2 * lane) =
                merge128(ov, __uint_as_float((uint32_t)ml), __uint_as_float((uint32_t)(ml >> 32)), &M, &inv);
        }
    };
    if (nw <= 8) merge_row(std::integral_constant<int, 8>{});
    else if (nw <= 16) merge_row(std::integral_constant<int, 16>{});
    else if (nw <= 32) merge_row(std::integral_constant<int, 32>{});
    else if (nw <= 64) merge_row(std::integral_constant<int, 64>{});
    else {  // more than 64 partials: chunks of 64, each merged unnormalised, folded into a running partial
        const int h = w;
        const float* p = prow0 + (int64_t)h * a.total_splits * (D + 2);
        float Mr = -INFINITY, Lr = 0.0f;
        float2 ar = {0.0f, 0.0f};
        for (int c0 = 0; c0 < nw; c0 += 64) {
            const int nc = min(64, nw - c0);
            float2 ov[64];
#pragma unroll
            for (int i = 0; i < 64; i++) {  // past the chunk's count: a counted row again, at weight 0
                const uint64_t v = __hip_atomic_load(
                    (const uint64_t*)(p + (int64_t)(c0 + min(i, nc - 1)) * (D + 2) + 2 * lane), __ATOMIC_RELAXED,
                    __HIP_MEMORY_SCOPE_AGENT);
                ov[i] = float2{__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32))};
            }
            uint64_t ml = 0xFF800000ull;
            if (lane < nc)
                ml = __hip_atomic_load((const uint64_t*)(p + (int64_t)(c0 + lane) * (D + 2) + D), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            float Mc, Lc;
            const float2 oc =
                merge128_partial(ov, __uint_as_float((uint32_t)ml), __uint_as_float((uint32_t)(ml >> 32)), &Mc, &Lc);
            fold_partial(Mr, Lr, ar, Mc, Lc, oc);
        }
        const float inv = Lr > 0.0f ? 1.0f / Lr : 0.0f;
        *(float2*)(a.out + ((int64_t)b * a.num_q_heads + kvh * G + h) * D + 2 * lane) = float2{ar.x * inv, ar.y * inv};
    }
}

// The one-launch step of a ragged batch (at most 64 sequences) in compact
// order: workgroup i's G waves take items G i .. G i + G - 1 of the compact
// order of split_append_kernel, so every wave slot holds a split with
// tokens.  The waves of a workgroup that share a row (KV head, entry) form
// a run of consecutive splits; each run is merged in LDS into one partial,
// written through to the workspace at the slot of its first split, and
// counted in the row's counter.  A row's runs are known from where its items
// start: a run begins at its split 0 and wherever an item index is a
// multiple of G.  The workgroup that counts a row's last run merges that
// row's run partials into the output.
template <int VB, int G>
__global__ __launch_bounds__(64 * G) __attribute__((amdgpu_waves_per_eu(2))) void split_append_merged_compact_kernel(
    MfmaArgs a)
{
    constexpr int D = 128;
    __shared__ uint4 meta_lds[G][META_BYTES / 16];
    __shared__ float part[G][G][D + 2];
    __shared__ int wrow[G], wsp[G], wnsp[G], wbase[G];
    __shared__ uint32_t ticket[G];
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int H = a.seg.f.H;
    // a row's runs: split 0, then every split whose item index is a multiple of G
    auto first_split = [](int base) { return G - base % G; };  // the second run's first split
    auto runs_of = [&](int base, int ns) {
        const int s1 = first_split(base);
        return s1 >= ns ? 1 : 2 + (ns - 1 - s1) / G;
    };
    {
        int sp, row, nsp;
        if (!compact_item(a, blockIdx.x * G, sp, row, nsp)) return;  // the whole group is past the last item
        const int lin = blockIdx.x * G + w;
        const bool has = compact_item(a, lin, sp, row, nsp);
        if (has) {
            split_body<VB, G, false, false, false, true, true>(a, sp, row % H, row / H, lane, meta_lds[w],
                                                                 &part[w][0][0]);
        } else if (lane < G) {  // past the last item
            part[w][lane][D] = -INFINITY;
            part[w][lane][D + 1] = 0.0f;
        }
        if (lane == 0) {
            wrow[w] = has ? row : -1;
            wsp[w] = sp;
            wnsp[w] = nsp;
            wbase[w] = lin - sp;  // the row's first item
        }
        __syncthreads();
        // runs: wave r starts one when its row differs from wave r - 1's; wave
        // w merges head w of every run
        for (int r = 0; r < G; r++) {
            const int rr = wrow[r];
            if (rr < 0 || (r > 0 && wrow[r - 1] == rr)) continue;
            int e = r + 1;
            while (e < G && wrow[e] == rr) e++;
            const int n = e - r, h = w;
            float2 ov[G];
#pragma unroll
            for (int i = 0; i < G; i++) ov[i] = *(const float2*)&part[min(r + i, e - 1)][h][2 * lane];
            const float mi = lane < n ? part[r + lane][h][D] : -INFINITY;
            const float li = lane < n ? part[r + lane][h][D + 1] : 0.0f;
            float M, L;
            const float2 o = merge128_partial(ov, mi, li, &M, &L);
            float* p = a.partials +
                       (((int64_t)(rr / H) * a.num_q_heads + (rr % H) * G + h) * a.total_splits + wsp[r]) * (D + 2);
            const uint64_t ob = (uint64_t)__float_as_uint(o.x) | ((uint64_t)__float_as_uint(o.y) << 32);
            __hip_atomic_store((uint64_t*)(p + 2 * lane), ob, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (lane == 0) {
                const uint64_t ml = (uint64_t)__float_as_uint(M) | ((uint64_t)__float_as_uint(L) << 32);
                __hip_atomic_store((uint64_t*)(p + D), ml, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's stores are complete
        __syncthreads();                                  // ... and every wave's
        if (lane == 0) {
            const int rr = wrow[w];
            uint32_t t = 0xFFFFFFFFu;
            if (rr >= 0 && (w == 0 || wrow[w - 1] != rr)) {
                const unsigned last = (unsigned)(runs_of(wbase[w], wnsp[w]) - 1);
                t = atomicInc(a.counters + rr, last) == last ? 1u : 0u;
            }
            ticket[w] = t;
        }
        __syncthreads();
        // rows whose last run this workgroup counted: wave w merges head w of
        // the row's run partials
        for (int r = 0; r < G; r++) {
            if (ticket[r] != 1u) continue;
            const int rr = wrow[r], nr = runs_of(wbase[r], wnsp[r]), s1 = first_split(wbase[r]), h = w;
            const float* p =
                a.partials + ((int64_t)(rr / H) * a.num_q_heads + (rr % H) * G + h) * a.total_splits * (D + 2);
            auto slot = [&](int j) { return j == 0 ? 0 : s1 + (j - 1) * G; };
            float Mr = -INFINITY, Lr = 0.0f;
            float2 ar = {0.0f, 0.0f};
            auto merge_runs = [&](auto ch) __attribute__((always_inline)) {
                constexpr int CH = decltype(ch)::value;
                for (int c0 = 0; c0 < nr; c0 += CH) {
                    const int nc = min(CH, nr - c0);
                    float2 ov[CH];
#pragma unroll
                    for (int i = 0; i < CH; i++) {  // past the count: a counted partial again, at weight 0
                        const uint64_t v = __hip_atomic_load(
                            (const uint64_t*)(p + (int64_t)slot(c0 + min(i, nc - 1)) * (D + 2) + 2 * lane),
                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        ov[i] = float2{__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32))};
                    }
                    uint64_t ml = 0xFF800000ull;
                    if (lane < nc)
                        ml = __hip_atomic_load((const uint64_t*)(p + (int64_t)slot(c0 + lane) * (D + 2) + D),
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    float Mc, Lc;
                    const float2 oc = merge128_partial(ov, __uint_as_float((uint32_t)ml),
                                                       __uint_as_float((uint32_t)(ml >> 32)), &Mc, &Lc);
                    fold_partial(Mr, Lr, ar, Mc, Lc, oc);
                }
            };
            if (nr <= 8) merge_runs(std::integral_constant<int, 8>{});
            else if (nr <= 16) merge_runs(std::integral_constant<int, 16>{});
            else merge_runs(std::integral_constant<int, 64>{});
            const float inv = Lr > 0.0f ? 1.0f / Lr : 0.0f;
            *(float2*)(a.out + ((int64_t)(rr / H) * a.num_q_heads + (rr % H) * G + h) * D + 2 * lane) =
                float2{ar.x * inv, ar.y * inv};
        }
    }
}

// Whether a segment has a matrix-core kernel.
static bool mfma_ok(const SegArgs& s, const void* q, int q_dtype, int32_t num_q_heads, float sm_scale,
                    int32_t split_tokens)
{
    const Fmt& f = s.f;
    const int G = num_q_heads / f.H;
    return q_dtype == LKV_BF16 && f.D == 128 && f.g == 64 && !f.fp16 && f.kb == 6 && (f.vb == 4 || f.vb == 6) &&
           (!f.k_norm || f.off_kn == f.off_ks + META_BYTES) &&  // the factors follow the metadata
           (G == 4 || G == 8) && ((uintptr_t)q & 15) == 0 &&  // Q is read 16 bytes at a time
           sm_scale > 0.0f &&                                   // the scale is applied after the block maximum
           split_tokens <= 64 * BT;  // a split's block-table entries are held one per lane
}

static MfmaArgs mfma_args(const SegArgs& s, const void* q, int32_t num_q_heads, float sm_scale, float tau_low,
                          int32_t split_tokens, int32_t total_splits, float* partials)
{
    MfmaArgs a;
    a.seg = s;
    a.q = (const uint16_t*)q;
    a.num_q_heads = num_q_heads;
    a.split_tokens = split_tokens;
    a.total_splits = total_splits;
    a.score_scale = sm_scale * 1.4426950408889634f;
    a.tau_low = tau_low;
    a.partials = partials;
    a.k_new = nullptr;
    a.v_new = nullptr;
    a.kv_dtype = 0;
    a.counters = nullptr;
    a.out = nullptr;
    a.items = 0;
    a.compact = 0;
    return a;
}

bool launch_decode_split_mfma_tiered(const SegArgs& high, const SegArgs& mid, const void* q, int q_dtype,
                                     int32_t batch, int32_t num_q_heads, float sm_scale, float tau_low,
                                     int32_t split_tokens, int32_t total_splits, float* partials,
                                     hipStream_t stream, hipError_t* err)
{
    if (high.f.vb != 6 || mid.f.vb != 4 || high.f.H != mid.f.H || high.f.k_norm || mid.f.k_norm ||
        !mfma_ok(high, q, q_dtype, num_q_heads, sm_scale, split_tokens) ||
        !mfma_ok(mid, q, q_dtype, num_q_heads, sm_scale, split_tokens))
        return false;
    *err = hipSuccess;
    if (batch == 0 || high.n_splits + mid.n_splits == 0) return true;  // nothing to launch
    const MfmaArgs a0 = mfma_args(high, q, num_q_heads, sm_scale, tau_low, split_tokens, total_splits, partials);
    const MfmaArgs a1 = mfma_args(mid, q, num_q_heads, sm_scale, tau_low, split_tokens, total_splits, partials);
    const int G = num_q_heads / high.f.H;
    dim3 grid((unsigned)(high.n_splits + mid.n_splits), (unsigned)high.f.H, (unsigned)batch);
    const bool dbg = high.skip_mask != nullptr;
    if (G == 4 && dbg) hipLaunchKernelGGL((split_mfma_tiered_kernel<4, true>), grid, dim3(64), 0, stream, a0, a1);
    else if (G == 4) hipLaunchKernelGGL((split_mfma_tiered_kernel<4, false>), grid, dim3(64), 0, stream, a0, a1);
    else if (dbg) hipLaunchKernelGGL((split_mfma_tiered_kernel<8, true>), grid, dim3(64), 0, stream, a0, a1);
    else hipLaunchKernelGGL((split_mfma_tiered_kernel<8, false>), grid, dim3(64), 0, stream, a0, a1);
    *err = hipGetLastError();
    return true;
}

template <bool DBG>
static void launch_pair(const MfmaArgs& a, int vb, bool kn, dim3 grid, hipStream_t st)
{
    if (vb == 4 && kn) hipLaunchKernelGGL((split_mfma_pair_kernel<4, true, DBG>), grid, dim3(64), 0, st, a);
    else if (vb == 4) hipLaunchKernelGGL((split_mfma_pair_kernel<4, false, DBG>), grid, dim3(64), 0, st, a);
    else if (kn) hipLaunchKernelGGL((split_mfma_pair_kernel<6, true, DBG>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((split_mfma_pair_kernel<6, false, DBG>), grid, dim3(64), 0, st, a);
}

template <bool DBG>
static void launch_multi8(const MfmaArgs& a, int vb, bool kn, dim3 grid, hipStream_t st)
{
    if (vb == 4 && kn) hipLaunchKernelGGL((split_mfma_multi8_kernel<4, true, DBG>), grid, dim3(64), 0, st, a);
    else if (vb == 4) hipLaunchKernelGGL((split_mfma_multi8_kernel<4, false, DBG>), grid, dim3(64), 0, st, a);
    else if (kn) hipLaunchKernelGGL((split_mfma_multi8_kernel<6, true, DBG>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((split_mfma_multi8_kernel<6, false, DBG>), grid, dim3(64), 0, st, a);
}

template <bool DBG>
static void launch_plain(const MfmaArgs& a, int vb, int G, bool kn, dim3 grid, hipStream_t st)
{
    if (kn) {  // direction-preserving K
        if (vb == 4 && G == 4) hipLaunchKernelGGL((split_mfma_kernel<4, 4, true, DBG>), grid, dim3(64), 0, st, a);
        else if (vb == 4) hipLaunchKernelGGL((split_mfma_kernel<4, 8, true, DBG>), grid, dim3(64), 0, st, a);
        else if (G == 4) hipLaunchKernelGGL((split_mfma_kernel<6, 4, true, DBG>), grid, dim3(64), 0, st, a);
        else hipLaunchKernelGGL((split_mfma_kernel<6, 8, true, DBG>), grid, dim3(64), 0, st, a);
    } else if (vb == 4 && G == 4) hipLaunchKernelGGL((split_mfma_kernel<4, 4, false, DBG>), grid, dim3(64), 0, st, a);
    else if (vb == 4) hipLaunchKernelGGL((split_mfma_kernel<4, 8, false, DBG>), grid, dim3(64), 0, st, a);
    else if (G == 4) hipLaunchKernelGGL((split_mfma_kernel<6, 4, false, DBG>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((split_mfma_kernel<6, 8, false, DBG>), grid, dim3(64), 0, st, a);
}

bool launch_append_decode_mfma(const SegArgs& s, const void* q, int q_dtype, int32_t batch, int32_t num_q_heads,
                               float sm_scale, float tau_low, int32_t split_tokens, int32_t total_splits,
                               float* partials, const void* k_new, const void* v_new, int kv_dtype,
                               hipStream_t stream, hipError_t* err, float* out, uint32_t* counters, bool ragged)
{
    const uintptr_t align = kv_dtype == LKV_F32 ? 8 : 4;  // a lane reads its two channels at once
    if (!mfma_ok(s, q, q_dtype, num_q_heads, sm_scale, split_tokens) || s.f.k_norm || s.q_per_seq != 1 ||
        s.skip_mask != nullptr || s.scores != nullptr || (uintptr_t)k_new % align != 0 ||
        (uintptr_t)v_new % align != 0)
        return false;
    const bool merge = counters != nullptr;
    const int G = num_q_heads / s.f.H;
    if (merge && ((s.n_splits + G - 1) / G > MERGED_MAX_PARTIALS || total_splits != s.n_splits || !out))
        return false;
    MfmaArgs a = mfma_args(s, q, num_q_heads, sm_scale, tau_low, split_tokens, total_splits, partials);
    a.k_new = k_new;
    a.v_new = v_new;
    a.kv_dtype = kv_dtype;
    a.counters = counters;
    a.out = out;
    a.compact = ragged && batch <= 64 ? batch : 0;
    if (merge && a.compact > 0) {  // compact order: one workgroup per G items (those past the last item return)
        const dim3 grid((unsigned)((s.n_splits * s.f.H * batch + G - 1) / G));
        auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(64 * G), 0, stream, a); };
        if (s.f.vb == 4 && G == 4) go(split_append_merged_compact_kernel<4, 4>);
        else if (s.f.vb == 4) go(split_append_merged_compact_kernel<4, 8>);
        else if (G == 4) go(split_append_merged_compact_kernel<6, 4>);
        else go(split_append_merged_compact_kernel<6, 8>);
    } else if (merge) {  // every (workgroup of G splits, KV head, entry), in the order above
        const dim3 grid((unsigned)((s.n_splits + G - 1) / G * s.f.H * batch));
        auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(64 * G), 0, stream, a, a); };
        if (s.f.vb == 4 && G == 4) go(split_append_merged_kernel<4, 4, false>);
        else if (s.f.vb == 4) go(split_append_merged_kernel<4, 8, false>);
        else if (G == 4) go(split_append_merged_kernel<6, 4, false>);
        else go(split_append_merged_kernel<6, 8, false>);
    } else {  // every (split, KV head, entry), in the order above (compact: every item fits, whatever the lengths)
        const dim3 grid((unsigned)(s.n_splits * s.f.H * batch));
        auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(64), 0, stream, a); };
        if (s.f.vb == 4 && G == 4) go(split_append_kernel<4, 4>);
        else if (s.f.vb == 4) go(split_append_kernel<4, 8>);
        else if (G == 4) go(split_append_kernel<6, 4>);
        else go(split_append_kernel<6, 8>);
    }
    *err = hipGetLastError();
    return true;
}

// The decode step of a tiered cache in one launch: HIGH (K6V6) takes the
// new rows, HIGH and MID (K6V4) are read, the splits are merged in the
// kernel.  false when the pair or the shape has no such kernel.
bool launch_append_decode_tiered_merged(const SegArgs& high, const SegArgs& mid, const void* q, int q_dtype,
                                        int32_t batch, int32_t num_q_heads, float sm_scale, float tau_low,
                                        int32_t split_tokens, int32_t total_splits, float* partials,
                                        const void* k_new, const void* v_new, int kv_dtype, hipStream_t stream,
                                        hipError_t* err, float* out, uint32_t* counters)
{
    const uintptr_t align = kv_dtype == LKV_F32 ? 8 : 4;  // a lane reads its two channels at once
    const int G = num_q_heads / high.f.H;
    if (high.f.vb != 6 || mid.f.vb != 4 || high.f.H != mid.f.H || high.f.k_norm || mid.f.k_norm ||
        !mfma_ok(high, q, q_dtype, num_q_heads, sm_scale, split_tokens) ||
        !mfma_ok(mid, q, q_dtype, num_q_heads, sm_scale, split_tokens) || high.q_per_seq != 1 ||
        mid.q_per_seq != 1 || high.skip_mask != nullptr || high.scores != nullptr || mid.skip_mask != nullptr ||
        mid.scores != nullptr || (uintptr_t)k_new % align != 0 || (uintptr_t)v_new % align != 0 || !out ||
        !counters || total_splits != high.n_splits + mid.n_splits ||
        (total_splits + G - 1) / G > MERGED_MAX_PARTIALS)
        return false;
    *err = hipSuccess;
    if (batch == 0) return true;
    MfmaArgs a0 = mfma_args(high, q, num_q_heads, sm_scale, tau_low, split_tokens, total_splits, partials);
    MfmaArgs a1 = mfma_args(mid, q, num_q_heads, sm_scale, tau_low, split_tokens, total_splits, partials);
    a0.k_new = k_new;
    a0.v_new = v_new;
    a0.kv_dtype = kv_dtype;
    a0.counters = a1.counters = counters;
    a0.out = a1.out = out;
    const dim3 grid((unsigned)((total_splits + G - 1) / G * high.f.H * batch));
    if (G == 4) hipLaunchKernelGGL((split_append_merged_kernel<6, 4, true>), grid, dim3(256), 0, stream, a0, a1);
    else hipLaunchKernelGGL((split_append_merged_kernel<6, 8, true>), grid, dim3(512), 0, stream, a0, a1);
    *err = hipGetLastError();
    return true;
}

// Returns true and launches when the format and shape have a matrix-core
// kernel; false leaves the call to the generic kernel.
bool launch_decode_split_mfma(const SegArgs& s, const void* q, int q_dtype, int32_t batch, int32_t num_q_heads,
                              float sm_scale, float tau_low, int32_t split_tokens, int32_t total_splits,
                              float* partials, hipStream_t stream, hipError_t* err)
{
    if (!mfma_ok(s, q, q_dtype, num_q_heads, sm_scale, split_tokens)) return false;
    const Fmt& f = s.f;
    const int G = num_q_heads / f.H;
    MfmaArgs a = mfma_args(s, q, num_q_heads, sm_scale, tau_low, split_tokens, total_splits, partials);
    const int T = s.q_per_seq;
    if (T > 1 && G == 4) {  // batch counts B * T entries: B * ceil(T / 2) pairs
        dim3 grid((unsigned)s.n_splits, (unsigned)f.H, (unsigned)(batch / T * ((T + 1) / 2)));
        if (s.skip_mask != nullptr) launch_pair<true>(a, f.vb, f.k_norm, grid, stream);
        else launch_pair<false>(a, f.vb, f.k_norm, grid, stream);
    } else if (T > 1) {  // 8 heads: a token's layout is full; the tokens of an item share its L2
        const int64_t items = (int64_t)s.n_splits * f.H * (batch / T);
        a.items = (int32_t)items;
        const dim3 grid((unsigned)((items + 7) / 8 * 8 * T));
        if (s.skip_mask != nullptr) launch_multi8<true>(a, f.vb, f.k_norm, grid, stream);
        else launch_multi8<false>(a, f.vb, f.k_norm, grid, stream);
    } else {
        dim3 grid((unsigned)s.n_splits, (unsigned)f.H, (unsigned)batch);
        if (s.skip_mask != nullptr) launch_plain<true>(a, f.vb, G, f.k_norm, grid, stream);
        else launch_plain<false>(a, f.vb, G, f.k_norm, grid, stream);
    }
    *err = hipGetLastError();
    return true;
}

}  // namespace lkv
