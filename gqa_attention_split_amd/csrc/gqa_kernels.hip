// Split-KV partial kernel and combine kernel for the GQA exp-sum-div graph on
// gfx950 (MI355X, CDNA4).
//
// Graph (Mirage GQA tutorial, "Mirage: Define GQA Computation Graph"):
//   A = Q K, E = exp(A), S = rowsum(E), O = (E / S) V   -- no scale, no max.
// Split-KV form (kaispace blog, sections 2.1 and 4.2-4.3: a for-loop over the
// key dimension that accumulates, then a combine block graph): a workgroup
// owns (batch row b, query tile, key chunk) and accumulates
//   W = sum_n P_n V[n]   and   L = sum_n P_n,   P_n = fp16(exp(a_n))
// over its chunk; O = sum_s W_s / sum_s L_s. With no running maximum the
// partials combine by plain sums.
//
// Partial kernel. A workgroup has QW x KS waves: QW query groups of 32*QT
// rows each, times KS key streams; stream ks takes every KS-th 32-key tile
// of the chunk. Per tile and wave:
//   * S^T = K^T Q^T on v_mfma_f32_32x32x16_f16: keys on the accumulator rows,
//     queries on its columns; Q^T stays in registers for the whole kernel.
//   * E = exp2(S') in fp32, where S' = (log2(e) Q) K comes from Q pre-scaled
//     once per workgroup; P = fp16(E) rounded to nearest even; L += P in fp32
//     (v_dot2_f32_f16 against (1, 1)). In the 32x32 accumulator layout a lane
//     holds 16 keys of one query in exactly the order the next MFMA's B
//     operand needs (two 16-key k-steps, 8 consecutive accumulator registers
//     each), so the scores never leave registers.
//   * O^T += V^T P^T on the same MFMA.
// K (head-dim-major), V (key-major) and Q are copied HBM -> LDS as they lie in
// memory by buffer_load ... lds, which moves no data through registers. The
// MFMA operands need the contraction index along each lane's 8 values, the
// slow index of both K and V tiles; ds_read_b64_tr_b16 delivers that
// transpose: within each group of 16 lanes it returns
// result[i][j] = source[4j + i/4][i % 4] over the 16 lanes' 4-element reads,
// i.e. lane i receives column i of a 4 x 16 block. LDS rows are XOR-swizzled
// at 32-byte granularity so that the four rows of such a block fall in
// distinct banks.
//
// Two ring disciplines:
//   * private (QW == 1): each wave owns its key stream and a two-tile LDS
//     ring; the loop has no workgroup barrier. A tile's operands are read into
//     registers first, which frees its buffer for the tile two ahead before
//     any of its MFMAs run.
//   * shared (QW > 1): the QW waves of a stream share each tile; a ring of
//     STAGES tiles per stream, one workgroup barrier per step, and a
//     three-phase software pipeline (first product of tile it, softmax of
//     it-1, second product of it-2).
// After the loop the KS streams of a query group are summed in LDS in a fixed
// order; with one split the kernel writes O = fp16(W / L), otherwise the
// normalised partial o_s = fp16(W / L) and L go to the caller's workspace for
// the combine kernel, which forms O = sum_s L_s o_s / sum_s L_s.
//
// Bounds. K/V/Q accesses go through buffer descriptors whose record count
// ends at the last valid byte of batch b's array (or at zero for tiles past
// the chunk end), so out-of-range lanes read zeros. K rows continue into the
// next row in memory, so in a tile that straddles N the lanes whose keys lie
// past N get an offset beyond the descriptor. Keys read as zero K columns and
// zero V rows have S = 0 and P = 1 and contribute nothing to W; they are
// counted and removed from L. Query rows past M are zero and never stored.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mga_internal.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x4 __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;

constexpr int KT = 32;                       // keys per tile
constexpr int K_ROW_BYTES = KT * 2;          // 64: one head dim's 32 keys
constexpr int LDS_LIMIT = 160 * 1024;
constexpr float LOG2E = 1.4426950408889634f;
constexpr int BUFFER_FLAGS = 0x00020000;     // gfx9 raw buffer descriptor, dword 3
constexpr uint32_t OOB = 0x80000000u;        // offset past every descriptor's records

constexpr int cmin(int a, int b) { return a < b ? a : b; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Tile geometry for head dim HD (64 or 128). A tile is 32 keys: the K part
// [HD d][32 keys] (64-byte rows) followed by the V part [32 keys][HD d].
template <int HD>
struct Geo {
    static_assert(HD == 64 || HD == 128, "head dim");
    static constexpr int V_ROW_BYTES = HD * 2;
    static constexpr int V_PART = KT * HD * 2;        // byte offset of the V part in a tile
    static constexpr int TILE_BYTES = 2 * V_PART;     // 8 KiB (HD 64) or 16 KiB (HD 128)
    static constexpr int Q_ROW_BYTES = HD * 2;
    static constexpr int RED_ROW_BYTES = HD * 4 + 16;  // fp32 row + 16-byte pad (bank spread)
    static constexpr int KSTEPS = HD / 16;            // 16-deep k-steps of the first product
    static constexpr int DT = HD / 32;                // 32-row blocks of O^T
    static constexpr int DMA = HD / 16;               // 1 KiB DMA instructions per tile part
    static constexpr int V_LPR = HD / 8;              // lanes per V row (16 bytes each)
    static constexpr int V_RPI = 64 / V_LPR;          // V rows per DMA instruction
    static_assert(V_RPI % 4 == 0, "V swizzle needs whole groups of four rows per instruction");
};

__device__ __forceinline__ half8 cat8(fp16x4 lo, fp16x4 hi) {
    const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(half8, u32x4{a.x, a.y, b.x, b.y});
}

__device__ __forceinline__ fp16x4 tr_read(const char *lds_byte_addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)(lds_byte_addr));
}

// K part: [64 d][32 keys] fp16, 64-byte rows of two 32-byte units; the unit
// index is XORed with bit 1 of the row.
__device__ __forceinline__ int k_off(int d, int col_byte) {
    return d * K_ROW_BYTES + (((col_byte >> 5) ^ ((d >> 1) & 1)) << 5) + (col_byte & 31);
}
// V part: [32 keys][HD d] fp16, rows of HD/16 32-byte units; the unit index
// is XORed with the row's low two bits.
template <int HD>
__device__ __forceinline__ int v_off(int key, int col_byte) {
    using G = Geo<HD>;
    return G::V_PART + key * G::V_ROW_BYTES + (((col_byte >> 5) ^ (key & 3)) << 5) + (col_byte & 31);
}

template <int HD, int QT, int QW, int KS>
struct Cfg {
    using G = Geo<HD>;
    static constexpr int TILE_BYTES = G::TILE_BYTES;
    static constexpr int NWAVES = QW * KS;
    static constexpr int ROWS = 32 * QT * QW;   // query rows per workgroup
    static_assert(G::DMA % QW == 0, "QW must divide the K and V DMA instructions of a tile");
    static_assert(KS >= 2, "streams");
    static constexpr int PER = G::DMA / QW;     // K (and V) DMA instructions per wave per tile
    static constexpr int TILE_OPS = 2 * PER;    // DMA instructions per wave per tile
    static constexpr bool PRIVATE = QW == 1;
    // Shared ring: each buffer holds one tile per stream; step `it` refills
    // the buffer of tile it-3, so DIST = STAGES - 3 tiles are in flight.
    static constexpr int STAGE_BYTES = KS * TILE_BYTES;
    static constexpr int STAGES = PRIVATE ? 2 : cmin(LDS_LIMIT / STAGE_BYTES, 10);
    static constexpr int DIST = PRIVATE ? 2 : STAGES - 3;
    static constexpr int RING_BYTES = PRIVATE ? NWAVES * 2 * TILE_BYTES : STAGES * STAGE_BYTES;
    // Q staging: past the private rings, or in shared-ring buffers that the
    // prologue leaves empty (DIST .. STAGES-1).
    static constexpr int Q_BYTES = ROWS * G::Q_ROW_BYTES;
    static constexpr int Q_OFF = PRIVATE ? RING_BYTES : DIST * STAGE_BYTES;
    static constexpr int Q_OPS = Q_BYTES / 1024;  // 1 KiB DMA instructions for the workgroup's Q
    static constexpr int RED_BYTES = 32 * QT * G::RED_ROW_BYTES + 32 * QT * 4;  // one wave's epilogue region
    static constexpr int LDS_BYTES = cmax(cmax(RING_BYTES, Q_OFF + Q_BYTES), NWAVES * RED_BYTES);
    static constexpr int DW = HD / KS;                // head dims each wave finalises
    static constexpr int VPL = 32 * QT * DW / 64;     // values per lane in the final write
    static_assert(PRIVATE || STAGES >= 5, "shared ring depth");
    static_assert(PRIVATE || Q_OFF + Q_BYTES <= RING_BYTES, "Q staging inside the free ring buffers");
    static_assert(LDS_BYTES <= LDS_LIMIT, "LDS budget");
    static_assert(DIST * TILE_OPS < 64, "vmcnt range");
    static_assert(VPL >= 4 && VPL % 4 == 0, "final write granularity");
};

// gfx9 raw buffer descriptor: 48-bit base, stride 0, `bytes` records, so
// that any offset at or past `bytes` reads zero. Built in SGPRs.
__device__ __forceinline__ i32x4 make_rsrc(const void *p, uint32_t bytes) {
    const uint64_t a = (uint64_t)p;
    i32x4 r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));
    r.z = __builtin_amdgcn_readfirstlane((int)bytes);
    r.w = BUFFER_FLAGS;
    return r;
}

// One buffer_load_dwordx4 ... lds: lane l's 16 bytes land at LDS byte
// address lds + 16 l. Issued through asm so that the compiler neither waits
// for these loads before unrelated LDS reads nor reorders memory accesses
// across them; completion is waited for explicitly (wait_vm / sync_tile).
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// ... then meet the other waves at the workgroup barrier.
template <int N>
__device__ __forceinline__ void sync_tile() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}
// Every LDS read this wave issued has returned.
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

// Per-lane DMA offsets of this wave's share of a tile (independent of the
// tile's position: the descriptor base moves instead). K instruction x fills
// K rows 16 r .. 16 r + 15 (r = qw*PER + x), 4 lanes per 64-byte row; V
// instruction x fills V rows V_RPI r .. V_RPI (r + 1) - 1, V_LPR lanes per
// row. A lane fetches the 16-byte unit that the row's swizzle puts at its
// position.
template <int HD, int QW>
struct TileDma {
    static constexpr int PER = Geo<HD>::DMA / QW;
    uint32_t koff[PER];  // byte offset of the lane's 8 keys of head dim d from the tile's key 0
    uint32_t kcol;       // first key of those 8, relative to the tile start
    uint32_t voff;       // byte offset within the tile's 32 x HD V block (instruction 0)
};
template <int HD, int QW>
__device__ __forceinline__ TileDma<HD, QW> make_tile_dma(int qw, int lane, int N) {
    using G = Geo<HD>;
    constexpr int PER = G::DMA / QW;
    TileDma<HD, QW> t;
    const uint32_t lc = (lane & 3) ^ (((lane >> 3) & 1) << 1);  // bit 1 of d = bit 3 of lane
    t.kcol = 8 * lc;
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const uint32_t d = 16 * (qw * PER + x) + (lane >> 2);
        t.koff[x] = (d * (uint32_t)N + t.kcol) * 2;
    }
    const uint32_t kr = G::V_RPI * (qw * PER) + lane / G::V_LPR;
    const uint32_t vc = (lane % G::V_LPR) ^ ((kr & 3) << 1);
    t.voff = (kr * HD + 8 * vc) * 2;
    return t;
}

// Issue this wave's DMA share of one stream's tile (keys key0 .. key0+31 of
// the batch whose K and V arrays start at kb and vb) into the LDS tile at
// byte address `lds`. `live` is false for tiles past the chunk end: their
// descriptors hold zero records and the tile fills with zeros without
// touching memory. The descriptors start at the tile and end with the batch.
template <int HD, int QW>
__device__ __forceinline__ void issue_tile(const _Float16 *kb, const _Float16 *vb, int N, int key0,
                                           bool live, uint32_t lds, int qw, const TileDma<HD, QW> &t) {
    constexpr int PER = Geo<HD>::DMA / QW;
    const int rem = N - key0;  // keys from key0 to the end of the batch (> 0 when live)
    const i32x4 kr = make_rsrc(kb + key0, live ? (uint32_t)(HD * N - key0) * 2 : 0u);
    const i32x4 vr = make_rsrc(vb + (size_t)key0 * HD, live ? (uint32_t)rem * (HD * 2) : 0u);
    const bool kin = (int)t.kcol < rem;
#pragma unroll
    for (int x = 0; x < PER; ++x) dma16(kr, kin ? t.koff[x] : OOB, lds + (qw * PER + x) * 1024);
#pragma unroll
    for (int x = 0; x < PER; ++x) dma16(vr, t.voff + x * 1024, lds + Geo<HD>::V_PART + (qw * PER + x) * 1024);
}

// Keys of a chunk of `len` keys that fall into this stream's first `nt` tiles
// (tile it of stream ks starts at key (it*KS + ks)*32 of the chunk).
template <int KS>
__device__ __forceinline__ int live_keys(int len, int ks, int nt) {
    const int full_tiles = len / KT, rem = len % KT;
    int live = full_tiles > ks ? KT * cmin(nt, (full_tiles - ks + KS - 1) / KS) : 0;
    if (rem != 0 && full_tiles >= ks && (full_tiles - ks) % KS == 0 && (full_tiles - ks) / KS < nt) live += rem;
    return live;
}

// Returns the LDS byte offset x (< 2^18) unchanged, but the compiler must
// assume it changed: used on a per-lane LDS base inside the loop so that it
// is not hoisted as base + each read's constant (one register and one add per
// read per step). The mask shows the value is non-negative, which lets each
// read's constant go into the instruction's offset field.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x & 0x3ffff;
}

// Per-lane LDS byte offsets (within a tile) of the transposed operand reads.
// The K part's swizzle depends on bit 1 of the row, which the +4 and +16 row
// steps leave unchanged, and the V part's on the row's low two bits, which
// the +8 and +16 row steps leave unchanged; so one base per read family
// plus immediate offsets covers every read.
template <int HD>
struct LaneOffsets {
    int k;                // K part, head dims 8h+jr (+4, +16 kk), keys 16 g1 + 4c
    int v[Geo<HD>::DT];   // V part, keys 4h+jr (+8, +16 t), head dims 32 dt + 16 g1 + 4c
};
template <int HD>
__device__ __forceinline__ LaneOffsets<HD> lane_offsets(int lane) {
    const int h = lane >> 5, g1 = (lane >> 4) & 1, jr = (lane & 15) >> 2, cb = 8 * (lane & 3);
    LaneOffsets<HD> r;
    r.k = k_off(8 * h + jr, 32 * g1 + cb);
#pragma unroll
    for (int dt = 0; dt < Geo<HD>::DT; ++dt) r.v[dt] = v_off<HD>(4 * h + jr, 64 * dt + 32 * g1 + cb);
    return r;
}

// A operands of the first product (K^T, HD/16 k-steps of 16) and of the
// second product (V^T: [t][dt] = keys 16t.., head dims 32dt..).
template <int HD>
__device__ __forceinline__ void read_k(const char *kb, half8 (&a)[Geo<HD>::KSTEPS]) {
#pragma unroll
    for (int kk = 0; kk < Geo<HD>::KSTEPS; ++kk)
        a[kk] = cat8(tr_read(kb + kk * 16 * K_ROW_BYTES), tr_read(kb + kk * 16 * K_ROW_BYTES + 4 * K_ROW_BYTES));
}
template <int HD>
__device__ __forceinline__ void read_v(const char *const (&vb)[Geo<HD>::DT], half8 (&a)[2][Geo<HD>::DT]) {
    constexpr int VR = Geo<HD>::V_ROW_BYTES;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int dt = 0; dt < Geo<HD>::DT; ++dt)
            a[t][dt] = cat8(tr_read(vb[dt] + t * 16 * VR), tr_read(vb[dt] + t * 16 * VR + 8 * VR));
}

// First product of one tile for one wave (32*QT queries): S^T = K^T Q^T.
template <int HD, int QT>
__device__ __forceinline__ void scores(const half8 (&a)[Geo<HD>::KSTEPS],
                                       const half8 (&qf)[QT][Geo<HD>::KSTEPS], float16v (&s)[QT]) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        s[qt] = float16v{};
#pragma unroll
        for (int kk = 0; kk < Geo<HD>::KSTEPS; ++kk)
            s[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[kk], qf[qt][kk], s[qt], 0, 0, 0);
    }
}

// Softmax numerators of one tile: E = exp2(S) (scores are in log2 units),
// P = fp16(E) rounded to nearest, L += P. In the 32x32 accumulator layout
// register r of lane l holds key 8*(r/4) + 4*(l/32) + r%4 of query l%32, so
// registers 8t..8t+7 are exactly the 8 k-slots of the second product's
// B operand for keys 16t..16t+15.
template <int QT>
__device__ __forceinline__ void softmax(const float16v (&s)[QT], half8 (&p)[QT][2], float (&lsum)[QT][2]) {
    const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float e0 = __builtin_amdgcn_exp2f(s[qt][8 * t + 2 * j]);
                const float e1 = __builtin_amdgcn_exp2f(s[qt][8 * t + 2 * j + 1]);
                const half2v hv = __builtin_convertvector(float2v{e0, e1}, half2v);
                p[qt][t][2 * j] = hv[0];
                p[qt][t][2 * j + 1] = hv[1];
                lsum[qt][t] = __builtin_amdgcn_fdot2(hv, ones, lsum[qt][t], false);
            }
        }
    }
}

// Second product of one tile: O^T += V^T P^T.
template <int HD, int QT>
__device__ __forceinline__ void pv(const half8 (&a)[2][Geo<HD>::DT], const half8 (&p)[QT][2],
                                   float16v (&oacc)[Geo<HD>::DT][QT]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int dt = 0; dt < Geo<HD>::DT; ++dt)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
                oacc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[t][dt], p[qt][t], oacc[dt][qt], 0, 0, 0);
}

template <int HD, int QT, int QW, int KS>
__global__ __launch_bounds__(64 * QW * KS) void gqa_partial_kernel(
    const _Float16 *__restrict__ q, const _Float16 *__restrict__ k,
    const _Float16 *__restrict__ v, _Float16 *__restrict__ o, _Float16 *__restrict__ ws_o,
    float *__restrict__ ws_l, int B, int M, int N, int chunk_keys, int nsplit, int mtiles) {
    using C = Cfg<HD, QT, QW, KS>;
    using G = Geo<HD>;
    constexpr int TILE_BYTES = G::TILE_BYTES, DT = G::DT, KSTEPS = G::KSTEPS;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

    // Workgroup -> (batch, split, query tile). Consecutive workgroup ids go to
    // different XCDs (id % 8); the query tiles of one (batch, split) pair get
    // ids 8 apart so they run on the same XCD and share its L2 copy of K/V.
    const int wid = blockIdx.x;
    const int pair = (wid / (8 * mtiles)) * 8 + (wid & 7);
    const int mtile = (wid >> 3) % mtiles;
    if (pair >= B * nsplit) return;  // whole workgroup: padding of the last group of 8
    const int b = pair / nsplit, split = pair - b * nsplit;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int qw = wave / KS, ks = wave - qw * KS;
    const int h = lane >> 5;

    const int kstart = split * chunk_keys;
    const int len = min(N, kstart + chunk_keys) - kstart;  // keys in this chunk (> 0)
    const int qrow0 = mtile * C::ROWS;                     // first query row of the workgroup
    const int qbase = qrow0 + qw * 32 * QT;                // first query row of this wave

    const _Float16 *kb = k + (size_t)b * HD * N;  // batch b's K [HD][N] and V [N][HD]
    const _Float16 *vb = v + (size_t)b * N * HD;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)(smem));
    const LaneOffsets<HD> lo = lane_offsets<HD>(lane);
    const TileDma<HD, QW> td = make_tile_dma<HD, QW>(qw, lane, N);

    // Tiles are numbered per stream: tile it of stream ks starts at chunk key
    // (it*KS + ks)*32. `ntiles` counts the tiles a stream visits.
    const int chunk_tiles = (len + KT - 1) / KT;
    const int ntiles = C::PRIVATE ? (chunk_tiles > ks ? (chunk_tiles - ks + KS - 1) / KS : 0)
                                  : (len + KS * KT - 1) / (KS * KT);
    auto tile_key = [&](int it) { return (it * KS + ks) * KT; };  // relative to kstart
    auto issue = [&](int it, uint32_t lds) {
        issue_tile<HD, QW>(kb, vb, N, kstart + tile_key(it), it < ntiles && tile_key(it) < len, lds, qw, td);
    };

    // Q for the workgroup's rows -> LDS (rows past M read zero). Issued before
    // any K/V tile so that the first step finds it.
    {
        const int qrows = min(C::ROWS, M - qrow0);
        const i32x4 qr = make_rsrc(q + ((size_t)b * M + qrow0) * HD, (uint32_t)qrows * G::Q_ROW_BYTES);
        for (int j = wave; j < C::Q_OPS; j += C::NWAVES)
            dma16(qr, (uint32_t)(j * 1024 + lane * 16), lds0 + C::Q_OFF + j * 1024);
    }

    float16v oacc[DT][QT];
    float lsum[QT][2];  // per lane: its 16 keys of every tile, two chains
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] = float16v{};
        lsum[qt][0] = 0.f;
        lsum[qt][1] = 0.f;
    }
    half8 qf[QT][KSTEPS];
    // Q^T fragments (B operand): lane holds query qbase + 32*qt + (lane & 31),
    // head dims 16*kk + 8*h .. +7, pre-scaled by log2(e) (fp32 product rounded
    // to fp16) so that the first product yields log2-domain scores and
    // E = exp2(S) needs no per-score multiply.
    auto load_q = [&]() {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const char *row = smem + C::Q_OFF + (qbase - qrow0 + 32 * qt + (lane & 31)) * G::Q_ROW_BYTES + 16 * h;
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                half8 x = *reinterpret_cast<const half8 *>(row + 32 * kk);
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = (_Float16)((float)x[j] * LOG2E);
                qf[qt][kk] = x;
            }
        }
        wait_lds();
    };

    if constexpr (C::PRIVATE) {
        // Wave-private ring: buffers ring0 and ring0 + TILE_BYTES.
        const uint32_t ring0 = lds0 + wave * 2 * TILE_BYTES;
        const char *ring = smem + wave * 2 * TILE_BYTES;
        issue(0, ring0);
        issue(1, ring0 + TILE_BYTES);
        sync_tile<2 * C::TILE_OPS>();  // this wave's Q share landed; barrier: all of Q landed
        load_q();
        for (int it = 0; it < ntiles; ++it) {
            wait_vm<C::TILE_OPS>();  // tile it landed (tile it+1 may still be in flight)
            const char *buf = ring + (it & 1) * TILE_BYTES;
            half8 ka[KSTEPS], va[2][DT];
            const char *vbase[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) vbase[dt] = buf + lo.v[dt];
            read_k<HD>(buf + lo.k, ka);
            read_v<HD>(vbase, va);
            wait_lds();              // the buffer is free: refill it with tile it+2
            issue(it + 2, ring0 + (it & 1) * TILE_BYTES);
            float16v s[QT];
            half8 p[QT][2];
            scores<HD, QT>(ka, qf, s);
            softmax<QT>(s, p, lsum);
            pv<HD, QT>(va, p, oacc);
        }
        wait_vm<0>();
        __syncthreads();  // every ring and the Q staging are free for the reduction
    } else {
        constexpr int STAGES = C::STAGES, DIST = C::DIST, SB = C::STAGE_BYTES;
        int fill_buf = 0;  // buffer receiving the next issued tile
        int fill_it = 0;   // next tile to issue
        auto issue_next = [&]() {
            issue(fill_it, lds0 + fill_buf * SB + ks * TILE_BYTES);
            fill_buf = fill_buf + 1 == STAGES ? 0 : fill_buf + 1;
            ++fill_it;
        };
        for (int j = 0; j < DIST; ++j) issue_next();
        sync_tile<DIST * C::TILE_OPS>();  // this wave's Q share landed; barrier: all of Q landed
        load_q();                        // done before the first refill overwrites the staging

        // Unsigned index arithmetic lets the compiler fold each read's constant
        // part into the LDS instruction's offset field.
        auto tile_at = [&](int it) {
            return smem + ((unsigned)it % (unsigned)STAGES) * (unsigned)SB + (unsigned)ks * (unsigned)TILE_BYTES;
        };
        auto sync = [&]() {
            sync_tile<(DIST - 1) * C::TILE_OPS>();  // tile it landed for every wave; its refill target is free
            issue_next();
        };
        // Step `it` runs the first product of tile it, the softmax numerators
        // of tile it-1 and the second product of tile it-2. The three are
        // independent, so each wave's instruction stream always holds both
        // MFMA and VALU work. The second product runs first in a step, so the
        // softmax of the same step may overwrite the weights p it consumed;
        // the scores alternate between s0 and s1.
        float16v s0[QT], s1[QT];
        half8 p[QT][2];
        auto g1 = [&](int it, float16v (&sv)[QT]) {
            half8 a[KSTEPS];
            read_k<HD>(tile_at(it) + opaque(lo.k), a);
            scores<HD, QT>(a, qf, sv);
        };
        auto sm = [&](const float16v (&sv)[QT]) { softmax<QT>(sv, p, lsum); };
        auto g2 = [&](int it) {
            half8 a[2][DT];
            const char *vbase[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) vbase[dt] = tile_at(it) + opaque(lo.v[dt]);
            read_v<HD>(vbase, a);
            pv<HD, QT>(a, p, oacc);
        };
        const int niter = ntiles;
        sync();                 // step 0
        g1(0, s0);
        sync();                 // step 1 (tile 1 may lie past the chunk: zeros, unused)
        g1(1, s1);
        sm(s0);
        int it = 2;
        for (; it + 1 < niter; it += 2) {
            sync();
            g2(it - 2);
            g1(it, s0);
            sm(s1);
            sync();
            g2(it - 1);
            g1(it + 1, s1);
            sm(s0);
        }
        if (it < niter) {       // one more full step, it even
            sync();
            g2(it - 2);
            g1(it, s0);
            sm(s1);
            ++it;
        }
        // Drain: tiles niter-2 and niter-1 still need their second product,
        // tile niter-1 its softmax (niter == 1: only tile 0's product).
        if (niter == 1) {
            g2(0);
        } else if (it & 1) {    // last step even: tile niter-1's scores in s0
            g2(niter - 2);
            sm(s0);
            g2(niter - 1);
        } else {                // last step odd: tile niter-1's scores in s1
            g2(niter - 2);
            sm(s1);
            g2(niter - 1);
        }
        sync_tile<0>();  // no DMA in flight, every wave done with the ring
    }

    // Keys of this stream's tiles that lie outside the chunk or past N read
    // as zeros and entered L as P = 1 each.
    const float masked = (float)(KT * ntiles - live_keys<KS>(len, ks, ntiles));

    // Sum the KS streams of each query group in LDS (fixed order), then
    // write O (one split) or the partial W, L.
    {
        char *reg = smem + wave * C::RED_BYTES;
        float *lreg = (float *)(reg + 32 * QT * G::RED_ROW_BYTES);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const int qr = 32 * qt + (lane & 31);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int d = 32 * dt + 8 * rb + 4 * h;
                    *(float4v *)(reg + qr * G::RED_ROW_BYTES + d * 4) =
                        float4v{oacc[dt][qt][4 * rb], oacc[dt][qt][4 * rb + 1], oacc[dt][qt][4 * rb + 2],
                                oacc[dt][qt][4 * rb + 3]};
                }
            const float mine = lsum[qt][0] + lsum[qt][1];
            const float lfull = mine + __shfl_xor(mine, 32) - masked;
            if (h == 0) lreg[qr] = lfull;
        }
    }
    __syncthreads();
    {
        const int qr = lane % (32 * QT);
        const int d0 = ks * C::DW + (lane / (32 * QT)) * C::VPL;
        float acc[C::VPL];
#pragma unroll
        for (int x = 0; x < C::VPL; ++x) acc[x] = 0.f;
        float l = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            const char *reg = smem + (qw * KS + s2) * C::RED_BYTES;
            const float *lreg = (const float *)(reg + 32 * QT * G::RED_ROW_BYTES);
#pragma unroll
            for (int x = 0; x < C::VPL; x += 4) {
                const float4v t = *(const float4v *)(reg + qr * G::RED_ROW_BYTES + (d0 + x) * 4);
                acc[x] += t[0];
                acc[x + 1] += t[1];
                acc[x + 2] += t[2];
                acc[x + 3] += t[3];
            }
            l += lreg[qr];
        }
        const int row = qbase + qr;
        if (row < M) {
            if (nsplit == 1) {
                _Float16 *dst = o + ((size_t)b * M + row) * HD + d0;
#pragma unroll
                for (int x = 0; x < C::VPL; x += 4) {
                    half4 hv;
#pragma unroll
                    for (int y = 0; y < 4; ++y) hv[y] = (_Float16)(acc[x + y] / l);
                    *(half4 *)(dst + x) = hv;
                }
            } else {
                // Normalised partial: o_s = fp16(W_s / L_s), L_s in fp32 (0 when
                // no weight survived fp16, so that it drops out of the combine).
                const size_t prow = ((size_t)split * B + b) * M + row;
                _Float16 *dst = ws_o + prow * HD + d0;
                const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
                for (int x = 0; x < C::VPL; x += 4) {
                    half4 hv;
#pragma unroll
                    for (int y = 0; y < 4; ++y) hv[y] = (_Float16)(acc[x + y] * inv);
                    *(half4 *)(dst + x) = hv;
                }
                if (ks == 0 && d0 == 0) ws_l[prow] = l;
            }
        }
    }
}

// Combine: HD/4 threads per output row, 4 head dims each.
// O = fp16(sum_s L_s o_s / sum_s L_s), both sums in split order.
template <int HD>
__global__ __launch_bounds__(256) void gqa_combine_kernel(const _Float16 *__restrict__ ws_o,
                                                          const float *__restrict__ ws_l,
                                                          _Float16 *__restrict__ o, long long rows,
                                                          int nsplit) {
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long row = gid / (HD / 4);
    const int c = (int)(gid % (HD / 4));
    if (row >= rows) return;
    float l = 0.f;
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) {
        const long long prow = (long long)s * rows + row;
        const float ls = ws_l[prow];
        const half4 os = *reinterpret_cast<const half4 *>(ws_o + prow * HD + 4 * c);
        l += ls;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += ls * (float)os[i];
    }
    half4 hv;
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = (_Float16)(acc[i] / l);
    *reinterpret_cast<half4 *>(o + row * HD + 4 * c) = hv;
}

template <int HD, int QT, int QW, int KS>
int launch_partial_cfg(const mga::Plan &p, const _Float16 *q, const _Float16 *k, const _Float16 *v,
                       _Float16 *o, _Float16 *w, float *l, hipStream_t st) {
    static_assert(32 * QT * QW == 32 || 32 * QT * QW == 64 || 32 * QT * QW == 128 || 32 * QT * QW == 256,
                  "rows per workgroup");
    const int pairs = p.B * p.splits;
    const int groups = (pairs + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * p.mtiles));
    hipLaunchKernelGGL((gqa_partial_kernel<HD, QT, QW, KS>), grid, dim3(64 * QW * KS), 0, st, q, k, v, o,
                       w, l, p.B, p.M, p.N, p.chunk_keys, p.splits, p.mtiles);
    return (int)hipGetLastError();
}

}  // namespace

namespace mga {

// Workspace: o_s [splits][B][M][D] fp16, then (from a 256-byte boundary)
// L_s [splits][B][M] fp32.
static void ws_split(const Plan &p, const void *ws, _Float16 **w, float **l) {
    const size_t rows = (size_t)p.splits * p.B * p.M;
    *w = (_Float16 *)ws;
    *l = (float *)((char *)ws + ((rows * p.D * sizeof(_Float16) + 255) & ~(size_t)255));
}

int launch_partial(const Plan &p, const void *q, const void *k, const void *v, void *o,
                   void *ws, void *stream) {
    _Float16 *w = nullptr;
    float *l = nullptr;
    if (p.splits > 1) ws_split(p, ws, &w, &l);
    hipStream_t st = (hipStream_t)stream;
    const _Float16 *qh = (const _Float16 *)q, *kh = (const _Float16 *)k, *vh = (const _Float16 *)v;
    _Float16 *oh = (_Float16 *)o;
    switch (p.variant) {
    case kVariantDecode: return launch_partial_cfg<64, 1, 1, 8>(p, qh, kh, vh, oh, w, l, st);
    case kVariantSmall: return launch_partial_cfg<64, 2, 1, 8>(p, qh, kh, vh, oh, w, l, st);
    case kVariantMedium: return launch_partial_cfg<64, 2, 2, 4>(p, qh, kh, vh, oh, w, l, st);
    case kVariantLarge: return launch_partial_cfg<64, 2, 4, 2>(p, qh, kh, vh, oh, w, l, st);
    case kVariantDecode128: return launch_partial_cfg<128, 1, 1, 4>(p, qh, kh, vh, oh, w, l, st);
    default: return (int)hipErrorInvalidValue;
    }
}

int launch_combine(const Plan &p, void *o, const void *ws, void *stream) {
    _Float16 *w = nullptr;
    float *l = nullptr;
    ws_split(p, ws, &w, &l);
    const long long rows = (long long)p.B * p.M;
    const long long threads = rows * (p.D / 4);
    const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
    if (p.D == 128)
        hipLaunchKernelGGL(gqa_combine_kernel<128>, grid, dim3(kThreads), 0, (hipStream_t)stream, w, l,
                           (_Float16 *)o, rows, p.splits);
    else
        hipLaunchKernelGGL(gqa_combine_kernel<64>, grid, dim3(kThreads), 0, (hipStream_t)stream, w, l,
                           (_Float16 *)o, rows, p.splits);
    return (int)hipGetLastError();
}

}  // namespace mga
