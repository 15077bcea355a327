// append.hip -- quantise-and-pack append (built with -ffp-contract=off).
//
// One workgroup owns one (sequence, logical block, KV head) chunk for the
// call, so the channel-major V rows, whose 32-bit words hold several tokens,
// are merged and written without atomics.  Each wave quantises whole rows
// (one token's K or V): the group min / max is a wavefront reduction over the
// lanes holding the group, the codes go to LDS, and the workgroup then packs
// 32-bit words and writes them with coalesced stores.
#include <hip/hip_fp16.h>

#include "lkv_internal.h"
#include "quant_device.h"

namespace lkv {

struct AppendArgs {
    Fmt f;
    uint8_t* pool;
    const void* k;
    const void* v;
    const int32_t* cu_new;
    const int32_t* start_pos;
    const int32_t* block_table;
    int32_t max_blocks;
    int32_t nblk;    // logical blocks a sequence's new rows can touch
    int32_t dtype;
};

template <int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a)
{
    constexpr int VPL = D / 64;  // values per lane: channels lane + 64 * i
    const Fmt& f = a.f;
    const int b = blockIdx.x / a.nblk;
    const int i = blockIdx.x % a.nblk;
    const int kvh = blockIdx.y;
    const int row0 = a.cu_new[b];
    const int n = a.cu_new[b + 1] - row0;
    if (n <= 0) return;
    const int sp = a.start_pos[b];
    const int lb = sp / BT + i;
    const int p0 = max(sp, lb * BT);
    const int p1 = min(sp + n, lb * BT + BT);
    if (p0 >= p1) return;
    const int s0 = p0 - lb * BT, s1 = p1 - lb * BT;  // slots written by this call
    const int64_t blk = a.block_table[(int64_t)b * a.max_blocks + lb];
    uint8_t* ch = a.pool + (blk * f.H + kvh) * f.chunk;

    __shared__ uint16_t kc[BT][D];
    __shared__ uint16_t vc[BT][D];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    for (int r = wave; r < 2 * (s1 - s0); r += 4) {
        const int slot = s0 + (r >> 1);
        const bool is_v = r & 1;
        const int64_t in_row = (int64_t)(row0 + (lb * BT + slot - sp)) * f.H + kvh;
        const void* src = is_v ? a.v : a.k;
        const int bits = is_v ? f.vb : f.kb;
#pragma unroll
        for (int j = 0; j < VPL; j++) {
            const int d = lane + 64 * j;
            const float x = load_as_float(src, in_row * D + d, a.dtype);
            uint32_t code;
            if (f.fp16) {
                code = f16_bits(x);
            } else {
                float s;
                int z;
                code = (uint32_t)quantize_lane(x, f.g, bits, &s, &z);
                if ((d % f.g) == 0) {
                    const int gi = d / f.g;
                    float* sc = (float*)(ch + (is_v ? f.off_vs : f.off_ks));
                    uint8_t* zc = ch + (is_v ? f.off_vz : f.off_kz);
                    sc[gi * BT + slot] = s;
                    zc[gi * BT + slot] = (uint8_t)z;
                }
            }
            if (is_v) vc[slot][d] = (uint16_t)code;
            else kc[slot][d] = (uint16_t)code;
        }
    }
    __syncthreads();

    // K rows: token-major, whole 32-bit words per token.
    const int wk = D * f.kb / 32;
    for (int idx = threadIdx.x; idx < (s1 - s0) * wk; idx += blockDim.x) {
        const int slot = s0 + idx / wk;
        const int w = idx % wk;
        const uint32_t word = pack_word(w, f.kb, 0, D, [&](int c) { return (uint32_t)kc[slot][c]; });
        ((uint32_t*)(ch + f.off_kc + slot * f.krow))[w] = word;
    }
    // V rows: channel-major; only the words that hold bits of slots [s0, s1)
    // are touched, and their bits of other slots are kept.
    const int w0 = (f.vb * s0) / 32, w1 = (f.vb * s1 - 1) / 32;
    const int wv = w1 - w0 + 1;
    for (int idx = threadIdx.x; idx < D * wv; idx += blockDim.x) {
        const int d = idx / wv;
        const int w = w0 + idx % wv;
        const uint32_t mask = field_mask(w, f.vb, s0, s1);
        uint32_t word = pack_word(w, f.vb, s0, s1, [&](int s) { return (uint32_t)vc[s][d]; });
        uint32_t* dst = (uint32_t*)(ch + f.off_vc + d * f.vrow) + w;
        if (mask != 0xFFFFFFFFu) word = (*dst & ~mask) | (word & mask);
        *dst = word;
    }
}

hipError_t launch_append(const Fmt& f, uint8_t* pool, const void* k, const void* v, int dtype,
                         const int32_t* cu_new, const int32_t* start_pos, const int32_t* block_table,
                         int32_t max_blocks, int32_t batch, int32_t max_new, hipStream_t stream)
{
    if (batch == 0 || max_new == 0) return hipSuccess;
    AppendArgs a;
    a.f = f;
    a.pool = pool;
    a.k = k;
    a.v = v;
    a.cu_new = cu_new;
    a.start_pos = start_pos;
    a.block_table = block_table;
    a.max_blocks = max_blocks;
    a.nblk = (max_new + BT - 1) / BT + 1;
    a.dtype = dtype;
    dim3 grid((unsigned)batch * (unsigned)a.nblk, (unsigned)f.H);
    if (f.D == 64) hipLaunchKernelGGL(append_kernel<64>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(append_kernel<128>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace lkv
