// append.hip -- quantise-and-pack append (built with -ffp-contract=off).
//
// append_quant_kernel serves the quantised formats; append_kernel the fp16
// format and inputs not aligned to two elements.
//
// One workgroup owns one (sequence, logical block, KV head) chunk for the
// call, so the channel-major V rows, whose 32-bit words hold several tokens,
// are merged and written without atomics.  Each wave quantises whole rows
// (one token's K or V): the group min / max is a wavefront reduction over the
// lanes holding the group, the codes go to LDS, and the workgroup then packs
// 32-bit words and writes them.
//
// Latency: every input load of a wave is issued before it quantises its
// first row, and the V words that other slots share are merged in memory
// with atomic AND/OR (no load of the old word), so a one-row decode append
// waits for two memory round trips: the indices, then the rows and the block
// table entry.
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
    int32_t len_cap; // cu_new null: start_pos holds lengths, clamped to this
};

// Input rows [row0, row0 + n) of sequence b go to positions sp, sp + 1, ...
// Without cu_new, each sequence appends one row (row b) at its last
// position: start_pos then holds the lengths, which count that row.
__device__ __forceinline__ void rows_of(const AppendArgs& a, int b, int& row0, int& n, int& sp)
{
    if (a.cu_new != nullptr) {
        row0 = a.cu_new[b];
        n = a.cu_new[b + 1] - row0;
        sp = a.start_pos[b];
    } else {
        row0 = b;
        sp = min(a.start_pos[b], a.len_cap) - 1;
        n = sp >= 0 ? 1 : 0;
    }
}

// Raw bits of input element i (fp32, or a 16-bit pattern), and their value.
template <int DT>
__device__ __forceinline__ uint32_t load_raw(const void* p, int64_t i)
{
    if constexpr (DT == LKV_F32) return ((const uint32_t*)p)[i];
    return ((const uint16_t*)p)[i];
}
template <int DT>
__device__ __forceinline__ float raw_value(uint32_t u)
{
    if constexpr (DT == LKV_F32) return __uint_as_float(u);
    if constexpr (DT == LKV_BF16) return __uint_as_float(u << 16);
    return __half2float(__ushort_as_half((uint16_t)u));
}

constexpr int MAXW = 16;  // V words per thread: D * 64 slots * 16 bits / 32 / 256 threads at most
constexpr int MAXR = 32;  // rows per wave: 64 slots x (K, V) / 4 waves
constexpr int CH = 8;     // rows whose loads are issued together

template <int D, int DT>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a)
{
    constexpr int VPL = D / 64;  // values per lane: channels lane + 64 * i
    const Fmt& f = a.f;
    const int b = blockIdx.x / a.nblk;
    const int i = blockIdx.x % a.nblk;
    const int kvh = blockIdx.y;
    // the index loads are independent: issued together
    int row0, n, sp;
    rows_of(a, b, row0, n, sp);
    const int lb = sp / BT + i;
    const int p0 = max(sp, lb * BT);
    const int p1 = min(sp + n, lb * BT + BT);
    if (n <= 0 || p0 >= p1) return;
    const int s0 = p0 - lb * BT, s1 = p1 - lb * BT;  // slots written by this call
    const int64_t blk = a.block_table[(int64_t)b * a.max_blocks + lb];
    uint8_t* ch = a.pool + (blk * f.H + kvh) * f.chunk;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
    const int nrows = 2 * (s1 - s0);  // row r: slot s0 + r / 2, K (r even) or V (r odd)

    __shared__ uint16_t kc[BT][D];
    __shared__ uint16_t vc[BT][D];
    // Rows go in chunks of CH per wave.  A chunk's input values are all
    // requested before any is used; rows past the end reload the last valid
    // row (in bounds, no branch), so the chunk waits for memory once.
#pragma unroll 1
    for (int k0 = 0; k0 < MAXR; k0 += CH) {
        if (wave + 4 * k0 >= nrows) break;
        uint32_t x[CH][VPL];  // raw bits: converted where used
#pragma unroll
        for (int k = 0; k < CH; k++) {
            const int r = min(wave + 4 * (k0 + k), nrows - 1);
            const int slot = s0 + (r >> 1);
            const int64_t in_row = (int64_t)(row0 + (lb * BT + slot - sp)) * f.H + kvh;
#pragma unroll
            for (int j = 0; j < VPL; j++) x[k][j] = load_raw<DT>((r & 1) ? a.v : a.k, in_row * D + lane + 64 * j);
        }
        auto process = [&](int k) {
            const int r = wave + 4 * (k0 + k);
            const int slot = s0 + (r >> 1);
            const bool is_v = r & 1;
            const int bits = is_v ? f.vb : f.kb;
#pragma unroll
            for (int j = 0; j < VPL; j++) {
                const int d = lane + 64 * j;
                uint32_t code;
                if (f.fp16) {
                    code = f16_bits(raw_value<DT>(x[k][j]));
                } else {
                    float sc;
                    int z;
                    code = (uint32_t)quantize_lane(raw_value<DT>(x[k][j]), f.g, bits, &sc, &z);
                    if ((d % f.g) == 0) {
                        const int gi = d / f.g;
                        float* scales = (float*)(ch + (is_v ? f.off_vs : f.off_ks));
                        uint8_t* zeros = ch + (is_v ? f.off_vz : f.off_kz);
                        scales[gi * BT + slot] = sc;
                        zeros[gi * BT + slot] = (uint8_t)z;
                    }
                }
                if (is_v) vc[slot][d] = (uint16_t)code;
                else kc[slot][d] = (uint16_t)code;
            }
        };
        if (wave + 4 * (k0 + CH - 1) < nrows) {
            // a full chunk: no branch between rows, so their independent
            // reductions and divisions interleave
#pragma unroll
            for (int k = 0; k < CH; k++) process(k);
        } else {
#pragma unroll
            for (int k = 0; k < CH; k++) {
                if (wave + 4 * (k0 + k) >= nrows) break;
                process(k);
            }
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
    // are written.  A word shared with other slots keeps their bits: its
    // field bits are cleared, then set, by two atomics (in program order to
    // the same address, so the second sees the first).
    const int w0 = (f.vb * s0) / 32, w1 = (f.vb * s1 - 1) / 32;
    const int wv = w1 - w0 + 1;
    const int nw = D * wv;
#pragma unroll
    for (int j = 0; j < MAXW; j++) {
        const int idx = threadIdx.x + 256 * j;
        if (idx < nw) {
            const int d = idx / wv, w = w0 + idx % wv;
            const uint32_t mask = field_mask(w, f.vb, s0, s1);
            const uint32_t word = pack_word(w, f.vb, s0, s1, [&](int s) { return (uint32_t)vc[s][d]; });
            uint32_t* dst = (uint32_t*)(ch + f.off_vc + d * f.vrow) + w;
            if (mask == 0xFFFFFFFFu) {
                *dst = word;
            } else {
                atomicAnd(dst, ~mask);
                atomicOr(dst, word & mask);
            }
        }
    }
}

// ---- quantised formats (K and V at 4 or 6 bits) ----
//
// The same placement as append_kernel, with each lane holding P = D / 64
// consecutive channels (one 4- or 8-byte load per lane and row), the faster
// quantiser, and word packing in whole groups of fields.  K codes are
// staged per slot (a lane's P codes in one 16-bit value), V codes channel-
// major with a row pitch of 68 bytes (the transposed stores of a wave hit
// distinct banks).
template <int DT, int P>
__device__ __forceinline__ void load_vals(const void* p, int64_t i, uint32_t (&u)[P])
{
    if constexpr (DT == LKV_F32) {
        if constexpr (P == 2) {
            const uint2 t = *(const uint2*)((const uint32_t*)p + i);
            u[0] = t.x;
            u[1] = t.y;
        } else {
            u[0] = ((const uint32_t*)p)[i];
        }
    } else {
        if constexpr (P == 2) {
            const uint32_t t = *(const uint32_t*)((const uint16_t*)p + i);
            u[0] = t & 0xFFFFu;
            u[1] = t >> 16;
        } else {
            u[0] = ((const uint16_t*)p)[i];
        }
    }
}

// K words of one slot: group m of NV lane values (NB bits each) -> NW words.
template <int NB, int NV, int NW>
__device__ __forceinline__ void pack_k_group(const uint16_t* row, int m, uint32_t* dst)
{
    uint32_t v[NV], w[NW];
#pragma unroll
    for (int i = 0; i < NV; i++) v[i] = row[m * NV + i];
    pack_values<NB, NV, NW>(v, w);
#pragma unroll
    for (int i = 0; i < NW; i++) dst[m * NW + i] = w[i];
}

template <int NB, int NV, int NW>
__device__ __forceinline__ void pack_k_rows(const uint16_t (*kq)[64], uint8_t* ch, const Fmt& f, int s0, int s1)
{
    constexpr int G = 64 / NV;  // groups per slot
    for (int idx = threadIdx.x; idx < (s1 - s0) * G; idx += blockDim.x) {
        const int slot = s0 + idx / G;
        pack_k_group<NB, NV, NW>(kq[slot], idx % G, (uint32_t*)(ch + f.off_kc + slot * f.krow));
    }
}

// Rows wave + 4 * (k0 + k), k < CHN, of one chunk: their loads are issued
// together, then they are quantised with their reductions interleaved (rows
// past the end reload the last row and are not stored).
template <int D, int DT, int CHN, int GS>
__device__ __forceinline__ void quant_rows(const AppendArgs& a, int k0, int wave, int lane, int nrows, int s0,
                                           int row0, int lb, int sp, int kvh, uint8_t* ch, uint16_t (*kq)[64],
                                           uint8_t (*vt)[VPITCH])
{
    constexpr int P = D / 64;
    const Fmt& f = a.f;
    uint32_t u[CHN][P];
#pragma unroll
    for (int k = 0; k < CHN; k++) {
        const int r = min(wave + 4 * (k0 + k), nrows - 1);
        const int slot = s0 + (r >> 1);
        const int64_t in_row = (int64_t)(row0 + (lb * BT + slot - sp)) * f.H + kvh;
        load_vals<DT, P>((r & 1) ? a.v : a.k, in_row * D + P * lane, u[k]);
    }
    QRow<P> q[CHN];
#pragma unroll
    for (int k = 0; k < CHN; k++) {
        const int r = wave + 4 * (k0 + k);
        float x[P];
#pragma unroll
        for (int p = 0; p < P; p++) x[p] = raw_value<DT>(u[k][p]);
        quantize_fast<P, GS>(x, (r & 1) ? f.vb : f.kb, q[k]);
    }
    // lanes whose quotient sat too close to a half-integer
#pragma unroll
    for (int k = 0; k < CHN; k++) {
        if (q[k].slow) {
            const int r = wave + 4 * (k0 + k);
            float x[P];
#pragma unroll
            for (int p = 0; p < P; p++) x[p] = raw_value<DT>(u[k][p]);
            quantize_exact<P>(x, (r & 1) ? f.vb : f.kb, q[k]);
        }
    }
    // direction-preserving K: the factor |k| / |k_hat| of each K row (rows of
    // waves 0 and 2), norms summed in fp64
    float rn[CHN];
    if (f.k_norm && (wave & 1) == 0) {
#pragma unroll
        for (int k = 0; k < CHN; k++) {
            double nx = 0.0, nk = 0.0;
#pragma unroll
            for (int p = 0; p < P; p++) {
                const double x = (double)raw_value<DT>(u[k][p]);
                const double kh = (double)(q[k].q[p] - q[k].z) * (double)q[k].s;
                nx += x * x;
                nk += kh * kh;
            }
            for (int o = 32; o > 0; o >>= 1) {
                nx += __shfl_xor(nx, o, 64);
                nk += __shfl_xor(nk, o, 64);
            }
            rn[k] = nk > 0.0 ? (float)sqrt(nx / nk) : 1.0f;
        }
    }
#pragma unroll
    for (int k = 0; k < CHN; k++) {
        const int r = wave + 4 * (k0 + k);
        if (r >= nrows) break;
        const int slot = s0 + (r >> 1);
        const bool is_v = r & 1;
        if (is_v) {
#pragma unroll
            for (int p = 0; p < P; p++) vt[P * lane + p][slot] = (uint8_t)q[k].q[p];
        } else {
            kq[slot][lane] = (uint16_t)(P == 2 ? (q[k].q[0] | (q[k].q[1] << f.kb)) : q[k].q[0]);
            if (f.k_norm && lane == 0) ((float*)(ch + f.off_kn))[slot] = rn[k];
        }
        if ((P * lane) % GS == 0) {
            const int gi = P * lane / GS;
            ((float*)(ch + (is_v ? f.off_vs : f.off_ks)))[gi * BT + slot] = q[k].s;
            ch[(is_v ? f.off_vz : f.off_kz) + gi * BT + slot] = (uint8_t)q[k].z;
        }
    }
}

template <int D, int DT, int GS>
__global__ __launch_bounds__(256) void append_quant_kernel(AppendArgs a)
{
    constexpr int P = D / 64;  // channels P * lane + p
    const Fmt& f = a.f;
    const int b = blockIdx.x / a.nblk;
    const int i = blockIdx.x % a.nblk;
    const int kvh = blockIdx.y;
    int row0, n, sp;
    rows_of(a, b, row0, n, sp);
    const int lb = sp / BT + i;
    const int p0 = max(sp, lb * BT);
    const int p1 = min(sp + n, lb * BT + BT);
    if (n <= 0 || p0 >= p1) return;
    const int s0 = p0 - lb * BT, s1 = p1 - lb * BT;  // slots written by this call
    const int64_t blk = a.block_table[(int64_t)b * a.max_blocks + lb];
    uint8_t* ch = a.pool + (blk * f.H + kvh) * f.chunk;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nrows = 2 * (s1 - s0);  // row r: slot s0 + r / 2, K (r even) or V (r odd)

    __shared__ uint16_t kq[BT][64];
    __shared__ uint8_t vt[D][VPITCH];
    if (nrows <= 4) {  // at most one row per wave (a decode step): no batch of duplicates
        if (wave < nrows) quant_rows<D, DT, 1, GS>(a, 0, wave, lane, nrows, s0, row0, lb, sp, kvh, ch, kq, vt);
    } else {
#pragma unroll 1
        for (int k0 = 0; k0 < MAXR; k0 += CH) {
            if (wave + 4 * k0 >= nrows) break;
            quant_rows<D, DT, CH, GS>(a, k0, wave, lane, nrows, s0, row0, lb, sp, kvh, ch, kq, vt);
        }
    }
    __syncthreads();
    const int knb = P * f.kb;  // bits of one lane's K value
    if (knb == 12) pack_k_rows<12, 8, 3>(kq, ch, f, s0, s1);
    else if (knb == 8) pack_k_rows<8, 4, 1>(kq, ch, f, s0, s1);
    else if (knb == 6) pack_k_rows<6, 16, 3>(kq, ch, f, s0, s1);
    else pack_k_rows<4, 8, 1>(kq, ch, f, s0, s1);
    if (f.vb == 6) pack_v_rows<6, 16, 3, D>(vt, ch, f.off_vc, f.vrow, s0, s1);
    else pack_v_rows<4, 8, 1, D>(vt, ch, f.off_vc, f.vrow, s0, s1);
}

template <int D, int GS>
static void launch_quant(const AppendArgs& a, int dtype, dim3 grid, hipStream_t stream)
{
    if constexpr (GS <= D) {
        if (dtype == LKV_F32) hipLaunchKernelGGL((append_quant_kernel<D, LKV_F32, GS>), grid, dim3(256), 0, stream, a);
        else if (dtype == LKV_BF16)
            hipLaunchKernelGGL((append_quant_kernel<D, LKV_BF16, GS>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((append_quant_kernel<D, LKV_F16, GS>), grid, dim3(256), 0, stream, a);
    }
}

template <int D>
static void launch_d(const AppendArgs& a, int dtype, dim3 grid, hipStream_t stream)
{
    // the quantised kernel loads P = D / 64 elements per lane at once: it needs
    // K and V aligned to P elements
    const uintptr_t need = (uintptr_t)(D / 64) * (dtype == LKV_F32 ? 4 : 2);
    const bool aligned = (uintptr_t)a.k % need == 0 && (uintptr_t)a.v % need == 0;
    if (a.f.fp16 || !aligned) {
        if (dtype == LKV_F32) hipLaunchKernelGGL((append_kernel<D, LKV_F32>), grid, dim3(256), 0, stream, a);
        else if (dtype == LKV_BF16) hipLaunchKernelGGL((append_kernel<D, LKV_BF16>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((append_kernel<D, LKV_F16>), grid, dim3(256), 0, stream, a);
        return;
    }
    if (a.f.g == 64) launch_quant<D, 64>(a, dtype, grid, stream);
    else if (a.f.g == 32) launch_quant<D, 32>(a, dtype, grid, stream);
    else launch_quant<D, 16>(a, dtype, grid, stream);
}

hipError_t launch_append(const Fmt& f, uint8_t* pool, const void* k, const void* v, int dtype,
                         const int32_t* cu_new, const int32_t* start_pos, const int32_t* block_table,
                         int32_t max_blocks, int32_t batch, int32_t max_new, hipStream_t stream, int32_t len_cap)
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
    a.len_cap = len_cap;
    dim3 grid((unsigned)batch * (unsigned)a.nblk, (unsigned)f.H);
    if (f.D == 64) launch_d<64>(a, dtype, grid, stream);
    else launch_d<128>(a, dtype, grid, stream);
    return hipGetLastError();
}

}  // namespace lkv
