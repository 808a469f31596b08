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
//     two-stage software pipeline: step it runs the first product of tile it
//     and the second product of tile it-1, with the softmax of one of them
//     (64-row tiles: the two waves of each SIMD take opposite phases, and the
//     first query wave of each stream issues all of the stream's DMA).
// After the loop the KS streams of a query group are summed in LDS in a fixed
// order; with one split the kernel writes O = fp16(W / L), otherwise the
// normalised partial o_s = fp16(W / L) and L go to the caller's workspace for
// the combine kernel, which forms O = sum_s L_s o_s / sum_s L_s.
//
// Layouts. Every operand is addressed through element strides (Strides):
// Q, V and O rows have unit stride along the head dim; K is either
// head-dim-major (K[d][n], unit stride along keys: the tutorial's
// pre-transposed K) or key-major (K[n][d], e.g. the transposed view of a
// [keys][head dim] cache). Row and batch strides are multiples of 8 elements,
// so every 16-byte DMA unit is aligned; N itself is unrestricted.
//
// Bounds. K/V/Q accesses go through buffer descriptors whose record count
// ends at the last valid byte of batch b's rows from the tile on (or at zero
// for tiles past the chunk end), so key rows past N and query rows past M read
// zeros. In a head-dim-major K a row continues past key N into padding or the
// next row, which the tile holding key N reads. That tile (and any tile past
// the chunk) therefore has its scores masked: keys past the chunk end get
// E = 0 whatever K held there. Query rows past M are never stored.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <tuple>
#include <type_traits>
#include <utility>

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

// Key-major K part: [32 keys][HD d] fp16, rows of HD/8 16-byte units; the
// unit index is XORed with the key's low three bits, so that the eight keys
// one ds_read_b128 pass serves hit eight distinct bank groups.
template <int HD>
__device__ __forceinline__ int km_off(int key, int col_byte) {
    return key * (HD * 2) + (((col_byte >> 4) ^ (key & 7)) << 4) + (col_byte & 15);
}

template <int HD, int QT, int QW, int KS, bool QKN = false>
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
    // Shared ring: each buffer holds one tile per stream. Every wave is done
    // with tile it-2 after step it-1, so step `it` may refill its buffer
    // (DIST = STAGES - 2 tiles in flight); QT = 1 refills tile it-3's buffer
    // instead (STAGES - 3 in flight), which timed faster for that shape (one
    // tile more or fewer in flight was slower, measured cold on MI355X).
    // With QK normalisation the ring leaves room for the key-scale slots
    // (one stage fewer) and refills tile it-2's buffer.
    static constexpr int STAGE_BYTES = KS * TILE_BYTES;
    static constexpr int SCR_BYTES = QKN ? NWAVES * 128 : 0;
    static constexpr int STAGES = PRIVATE ? 2 : cmin((LDS_LIMIT - SCR_BYTES) / STAGE_BYTES, 10);
    static constexpr int DIST = PRIVATE ? 2 : QT == 1 && !QKN ? STAGES - 3 : STAGES - 2;
    static constexpr int RING_BYTES = PRIVATE ? NWAVES * 2 * TILE_BYTES : STAGES * STAGE_BYTES;
    // Q staging: past the private rings, or in shared-ring buffers that the
    // prologue leaves empty (DIST .. STAGES-1).
    static constexpr int Q_BYTES = ROWS * G::Q_ROW_BYTES;
    static constexpr int Q_OFF = PRIVATE ? RING_BYTES : DIST * STAGE_BYTES;
    static constexpr int Q_OPS = Q_BYTES / 1024;  // 1 KiB DMA instructions for the workgroup's Q
    // One wave's epilogue region: its W rows (fp32), L per row, and with QK
    // normalisation the running maximum per row.
    static constexpr int RED_BYTES = 32 * QT * G::RED_ROW_BYTES + 32 * QT * 4 * (QKN ? 2 : 1);
    // QK normalisation: 128 bytes per wave (SCR_BYTES) to move key scales
    // between lanes.
    static constexpr int SCR_OFF = cmax(cmax(RING_BYTES, Q_OFF + Q_BYTES), NWAVES * RED_BYTES);
    static constexpr int LDS_BYTES = SCR_OFF + SCR_BYTES;
    static_assert(!QKN || PRIVATE || QT == 1, "QK normalisation: wave-private ring or 32-row query waves");
    static constexpr int DW = HD / KS;                // head dims each wave finalises
    static constexpr int VPL = 32 * QT * DW / 64;     // values per lane in the final write
    static_assert(PRIVATE || STAGES >= (QKN ? 4 : 5), "shared ring depth");
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
// The asm sets m0 (the LDS destination) and lists it as clobbered; clang
// warns that it does not preserve reserved registers across asm. These
// kernels have no other m0 user (the generated code sets m0 only inside
// these asm blocks), so nothing live is lost.
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
// tile's position: the descriptor base moves instead). Instruction x of the
// wave fills 1 KiB of the K part and 1 KiB of the V part:
//   * head-dim-major K: K rows 16 r .. 16 r + 15 (r = qw*PER + x), 4 lanes
//     per 64-byte row of 32 keys;
//   * key-major K and V: key rows V_RPI r .. V_RPI (r + 1) - 1, V_LPR lanes
//     per row.
// A lane fetches the 16-byte unit that the row's swizzle puts at its
// position.
template <int HD, int QW>
struct TileDma {
    static constexpr int PER = Geo<HD>::DMA / QW;
    uint32_t koff[PER];  // byte offset of the lane's K unit from the tile's key 0
    uint32_t kcol;       // head-dim-major: first of the lane's 8 keys, relative to the tile
    uint32_t voff[PER];  // byte offset of the lane's V unit from the tile's key 0
};
template <int HD, int QW, bool KM>
__device__ __forceinline__ TileDma<HD, QW> make_tile_dma(int qw, int lane, int k_r, int v_n) {
    using G = Geo<HD>;
    constexpr int PER = G::DMA / QW;
    TileDma<HD, QW> t;
    const uint32_t lc = (lane & 3) ^ (((lane >> 3) & 1) << 1);  // bit 1 of d = bit 3 of lane
    t.kcol = 8 * lc;
    const uint32_t kr = G::V_RPI * (qw * PER) + lane / G::V_LPR;  // key row of instruction 0
    const uint32_t vc = (lane % G::V_LPR) ^ ((kr & 3) << 1);     // same for every x: V_RPI % 4 == 0
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        if constexpr (KM) {
            const uint32_t key = kr + x * G::V_RPI;
            t.koff[x] = (key * (uint32_t)k_r + 8 * ((lane % G::V_LPR) ^ (key & 7))) * 2;
        } else {
            const uint32_t d = 16 * (qw * PER + x) + (lane >> 2);
            t.koff[x] = (d * (uint32_t)k_r + t.kcol) * 2;
        }
        t.voff[x] = ((kr + x * G::V_RPI) * (uint32_t)v_n + 8 * vc) * 2;
    }
    return t;
}

// Issue this wave's DMA share of one stream's tile into the LDS tile at byte
// address `lds`. kp / vp point at the tile's first key in K and V; krec / vrec
// are the byte extents from there to the batch's last valid byte. `live` is
// false for a tile past the chunk end: its descriptors hold zero records and
// the tile fills with zeros without touching memory. Key rows past N read
// zeros; in a head-dim-major K a lane's 8 keys may run past N into the rest
// of the row (or the next row), which the tail mask discards.
template <int HD, int QW>
__device__ __forceinline__ void issue_tile(const _Float16 *kp, uint32_t krec, const _Float16 *vp, uint32_t vrec,
                                           bool live, uint32_t lds, int qw, const TileDma<HD, QW> &t) {
    constexpr int PER = Geo<HD>::DMA / QW;
    const i32x4 kr = make_rsrc(kp, live ? krec : 0u);
    const i32x4 vr = make_rsrc(vp, live ? vrec : 0u);
#pragma unroll
    for (int x = 0; x < PER; ++x) dma16(kr, t.koff[x], lds + (qw * PER + x) * 1024);
#pragma unroll
    for (int x = 0; x < PER; ++x) dma16(vr, t.voff[x], lds + Geo<HD>::V_PART + (qw * PER + x) * 1024);
}

// Returns p, a pointer into the kernel's LDS block (byte offset below 2^18),
// but the compiler must assume it changed: the per-lane base of a tile's
// operand reads (tile offset + lane offset) is formed once per step, and each
// read's constant goes into the instruction's unsigned offset field. Left to
// itself the compiler folds the tile offset and one read's constant into a
// scalar base, which leaves the other reads' constants negative: one add per
// read.
__device__ __forceinline__ const char *lds_base(const char *smem, const char *p) {
    uint32_t off = (uint32_t)(p - smem);
    asm volatile("" : "+v"(off));
    __builtin_assume(off < (1u << 18));
    return smem + off;
}

// Per-lane LDS byte offsets (within a tile) of the transposed operand reads.
// The K part's swizzle depends on bit 1 of the row, which the +4 and +16 row
// steps leave unchanged, and the V part's on the row's low two bits, which
// the +8 and +16 row steps leave unchanged; so one base per read family
// plus immediate offsets covers every read.
template <int HD>
struct LaneOffsets {
    int k;                // head-dim-major K part, head dims 8h+jr (+4, +16 kk), keys 16 g1 + 4c
    int v[Geo<HD>::DT];   // V part, keys 4h+jr (+8, +16 t), head dims 32 dt + 16 g1 + 4c
    int krow;             // key-major K part: byte offset of the lane's key row (key l % 32)
    int kx;               // key-major K part: h ^ (key & 7); k-step kk reads unit 2 kk ^ kx
};
template <int HD>
__device__ __forceinline__ LaneOffsets<HD> lane_offsets(int lane) {
    const int h = lane >> 5, g1 = (lane >> 4) & 1, jr = (lane & 15) >> 2, cb = 8 * (lane & 3);
    LaneOffsets<HD> r;
    r.k = k_off(8 * h + jr, 32 * g1 + cb);
    r.krow = (lane & 31) * (HD * 2);
    r.kx = h ^ (lane & 7);
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
// Key-major K: lane l needs key l % 32, head dims 16 kk + 8 h .. +7, i.e.
// logical unit 2 kk + h of its row, stored at unit (2 kk + h) ^ (key & 7)
// = 2 kk ^ kx.
template <int HD>
__device__ __forceinline__ void read_k_km(const char *tile, int krow, int kx, half8 (&a)[Geo<HD>::KSTEPS]) {
#pragma unroll
    for (int kk = 0; kk < Geo<HD>::KSTEPS; ++kk)
        a[kk] = *reinterpret_cast<const half8 *>(tile + krow + (((2 * kk) ^ kx) << 4));
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
// With MASK, keys of the tile at or past `lim` (tile-relative) get E = 0:
// register r holds key 8*(r/4) + 4*h + r%4, compared against lim - 4*h.
template <int QT, bool MASK>
__device__ __forceinline__ void softmax(const float16v (&s)[QT], half8 (&p)[QT][2], float (&lsum)[QT][2],
                                        int lim_h) {
    const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r0 = 8 * t + 2 * j, r1 = r0 + 1;
                float e0 = __builtin_amdgcn_exp2f(s[qt][r0]);
                float e1 = __builtin_amdgcn_exp2f(s[qt][r1]);
                if constexpr (MASK) {
                    e0 = 8 * (r0 / 4) + r0 % 4 < lim_h ? e0 : 0.f;
                    e1 = 8 * (r1 / 4) + r1 % 4 < lim_h ? e1 : 0.f;
                }
                const half2v hv = __builtin_convertvector(float2v{e0, e1}, half2v);
                p[qt][t][2 * j] = hv[0];
                p[qt][t][2 * j + 1] = hv[1];
                lsum[qt][t] = __builtin_amdgcn_fdot2(hv, ones, lsum[qt][t], false);
            }
        }
    }
}

// QK-normalised softmax numerators of one tile. Scores S = Q K arrive from raw
// Q and K (exact fp16 products, fp32 sums); a = S * rk * rq - m is the
// log2-domain normalised score of each key (rk: the key's 1/rms in
// accumulator layout; rq: log2(e) / rms of the lane's query row) relative to
// the row's reference maximum m. The normalised scores reach
// |a| <= D log2(e), far past fp16 for exp, so the row keeps a reference m
// (FlashAttention's running maximum, applied lazily): when a tile's largest
// score exceeds m by more than 8, or the row has no reference yet, m moves to
// that score and W, L are rescaled by 2^(m_old - m_new). P = fp16(2^a) then
// stays below 2^8. Both lanes of a query (l, l+32) hold the same m.
template <int DT, int QT, bool MASK>
__device__ __forceinline__ void softmax_qkn(const float16v (&s)[QT], const float16v &rk, const float (&rq)[QT],
                                            half8 (&p)[QT][2], float (&lsum)[QT][2], float (&m)[QT],
                                            bool (&real)[QT], float16v (&oacc)[DT][QT], int lim_h) {
    constexpr float TH = 8.f;
    const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        float a[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            a[r] = __builtin_fmaf(s[qt][r] * rk[r], rq[qt], -m[qt]);
            if constexpr (MASK) a[r] = 8 * (r / 4) + r % 4 < lim_h ? a[r] : -__builtin_inff();
        }
        float mx = a[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = __builtin_fmaxf(mx, a[r]);
        mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32));
        const bool need = mx > TH || (!real[qt] && mx > -__builtin_inff());
        if (__builtin_amdgcn_ballot_w64(need)) {
            const float delta = need ? mx : 0.f;
            // A row without a reference has W = L = 0: scale by 0, not 2^-delta.
            const float sc = need ? (real[qt] ? __builtin_amdgcn_exp2f(-delta) : 0.f) : 1.f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt][qt] *= sc;
            lsum[qt][0] *= sc;
            lsum[qt][1] *= sc;
            m[qt] += delta;
            real[qt] = real[qt] || need;
#pragma unroll
            for (int r = 0; r < 16; ++r) a[r] -= delta;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float e0 = __builtin_amdgcn_exp2f(a[8 * t + 2 * j]);
                const float e1 = __builtin_amdgcn_exp2f(a[8 * t + 2 * j + 1]);
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

template <int HD, int QT, int QW, int KS, bool KM, bool QKN>
__global__ __launch_bounds__(64 * QW * KS) void gqa_partial_kernel(
    const _Float16 *__restrict__ q, const _Float16 *__restrict__ k,
    const _Float16 *__restrict__ v, _Float16 *__restrict__ o, _Float16 *__restrict__ ws_o,
    float *__restrict__ ws_l, mga::Strides st, int B, int M, int N, int chunk_keys, int nsplit, int mtiles,
    float eps) {
    using C = Cfg<HD, QT, QW, KS, QKN>;
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

    const _Float16 *kb = k + b * st.k_b;  // batch b's K and V
    const _Float16 *vb = v + b * st.v_b;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)(smem));
    const LaneOffsets<HD> lo = lane_offsets<HD>(lane);
    const TileDma<HD, QW> td = make_tile_dma<HD, QW, KM>(qw, lane, st.k_r, st.v_n);
    // 32-row query waves on the shared ring: the first query wave of each
    // stream (the early wave of its SIMD, which waits at each step's barrier
    // for the late one) issues the stream's whole tile; the late wave issues
    // no DMA at all.
    constexpr bool ONE_ISSUER = !C::PRIVATE && QT == 1;
    constexpr int T1 = 2 * G::DMA;  // DMA instructions per tile of the issuing wave
    const bool early = wave < C::NWAVES / 2;
    [[maybe_unused]] const TileDma<HD, 1> td1 = make_tile_dma<HD, 1, KM>(0, lane, st.k_r, st.v_n);

    // Tiles are numbered per stream: tile it of stream ks starts at chunk key
    // (it*KS + ks)*32. `ntiles` counts the tiles a stream visits.
    const int chunk_tiles = (len + KT - 1) / KT;
    const int ntiles = C::PRIVATE ? (chunk_tiles > ks ? (chunk_tiles - ks + KS - 1) / KS : 0)
                                  : (len + KS * KT - 1) / (KS * KT);
    auto tile_key = [&](int it) { return (it * KS + ks) * KT; };  // relative to kstart
    // Tile cursor of this stream: descriptor bases and byte extents of the
    // next tile to issue. Tiles are issued in order, KS*32 keys apart, so the
    // cursor advances by constant steps; `nlive` counts the stream's tiles
    // that start inside the chunk.
    const int key_first = kstart + ks * KT;
    const int rem0 = N - key_first;  // > 0 whenever nlive > 0
    const int nlive = len > ks * KT ? (len - ks * KT + KS * KT - 1) / (KS * KT) : 0;
    const long long kstep = KM ? (long long)KS * KT * st.k_r : (long long)KS * KT;  // elements
    const long long vstep = (long long)KS * KT * st.v_n;
    const _Float16 *kcur = kb + (KM ? (long long)key_first * st.k_r : (long long)key_first);
    const _Float16 *vcur = vb + (long long)key_first * st.v_n;
    // Head-dim-major K: the extent ends with the 16-byte unit holding the
    // batch's last key in row HD-1 (the unit lies in the row's storage, which
    // starts 16-byte aligned), so a lane whose 8 keys straddle N reads its
    // live keys whatever the granularity of the hardware's range check.
    uint32_t krec = KM ? ((uint32_t)(rem0 - 1) * (uint32_t)st.k_r + HD) * 2
                       : ((uint32_t)(HD - 1) * (uint32_t)st.k_r + (((uint32_t)rem0 + 7) & ~7u)) * 2;
    uint32_t vrec = ((uint32_t)(rem0 - 1) * (uint32_t)st.v_n + HD) * 2;
    const uint32_t krec_step = (uint32_t)kstep * 2, vrec_step = (uint32_t)vstep * 2;
    auto issue = [&](int it, uint32_t lds) {  // called for it = 0, 1, 2, ... in order
        if constexpr (ONE_ISSUER) {
            if (early) issue_tile<HD, 1>(kcur, krec, vcur, vrec, it < nlive, lds, 0, td1);
        } else {
            issue_tile<HD, QW>(kcur, krec, vcur, vrec, it < nlive, lds, qw, td);
        }
        kcur += kstep;
        vcur += vstep;
        krec -= krec_step;
        vrec -= vrec_step;
    };

    // Q for the workgroup's rows -> LDS rows of HD*2 bytes (rows past M read
    // zero). Issued before any K/V tile so that the first step finds it. The
    // 16-byte units of row r are XORed with r & 7: the operand reads take one
    // unit of 32 consecutive rows, which then fall in distinct banks.
    {
        constexpr int QLPR = HD / 8, QRPI = 64 / QLPR;  // lanes per row, rows per instruction
        const int qrows = min(C::ROWS, M - qrow0);
        const i32x4 qr = make_rsrc(q + b * st.q_b + (size_t)qrow0 * st.q_i,
                                   ((uint32_t)(qrows - 1) * (uint32_t)st.q_i + HD) * 2);
        const uint32_t lrow = lane / QLPR, lunit = lane % QLPR;
        for (int j = wave; j < C::Q_OPS; j += C::NWAVES) {
            const uint32_t row = j * QRPI + lrow;
            dma16(qr, row * (uint32_t)st.q_i * 2 + 16 * (lunit ^ (row & 7)), lds0 + C::Q_OFF + j * 1024);
        }
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
    // With QK normalisation Q stays unscaled (exact in the first product, whose
    // scores reach |D| after normalisation, where an fp16 rounding of the
    // scaled Q would show); rq gets log2(e) / rms of the lane's query row, the
    // sum of squares taken in fp32 over the lane's D/2 entries and its partner
    // lane's (l ^ 32).
    [[maybe_unused]] float rq[QT];
    auto load_q = [&]() {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const int r = qbase - qrow0 + 32 * qt + (lane & 31);  // staging row
            const char *row = smem + C::Q_OFF + r * G::Q_ROW_BYTES;
            half8 x[KSTEPS];
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk)  // head dims 16kk + 8h ..: unit 2kk + h, swizzled
                x[kk] = *reinterpret_cast<const half8 *>(row + 16 * ((2 * kk + h) ^ (r & 7)));
            if constexpr (QKN) {
                float ss = 0.f;
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
                    for (int j = 0; j < 8; j += 2) {
                        const half2v pr = {x[kk][j], x[kk][j + 1]};
                        ss = __builtin_amdgcn_fdot2(pr, pr, ss, false);
                    }
                ss += __shfl_xor(ss, 32);
                rq[qt] = LOG2E * __builtin_amdgcn_rsqf(ss * (1.f / HD) + eps);
            } else {
#pragma unroll
                for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
                    for (int j = 0; j < 8; ++j) x[kk][j] = (_Float16)((float)x[kk][j] * LOG2E);
            }
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) qf[qt][kk] = x[kk];
        }
        wait_lds();
    };

    // QK normalisation: 1/rms of each key of a tile, in the accumulator layout
    // of the scores (register r of lane l <-> key 8(r/4) + 4(l/32) + r%4). The
    // sum of squares comes in fp32 from the K^T operand (lane l: key l%32, D/2
    // entries; partner lane l ^ 32 the rest), then goes through this wave's
    // 32-float LDS slot to the lanes that hold the key's scores.
    [[maybe_unused]] float m_run[QT];
    [[maybe_unused]] bool real[QT];
    if constexpr (QKN) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            m_run[qt] = 0.f;
            real[qt] = false;
        }
    }
    auto scales_from_slot = [&](const float *slot, float16v &rk) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4v t = *reinterpret_cast<const float4v *>(slot + 8 * g + 4 * h);
            rk[4 * g] = t[0];
            rk[4 * g + 1] = t[1];
            rk[4 * g + 2] = t[2];
            rk[4 * g + 3] = t[3];
        }
    };
    auto key_scales_at = [&](const half8 (&ka)[KSTEPS], float16v &rk, float *slot) {
        float ss = 0.f;
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk)
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                const half2v pr = {ka[kk][j], ka[kk][j + 1]};
                ss = __builtin_amdgcn_fdot2(pr, pr, ss, false);
            }
        ss += __shfl_xor(ss, 32);
        const float r = __builtin_amdgcn_rsqf(ss * (1.f / HD) + eps);
        if (h == 0) slot[lane & 31] = r;
        scales_from_slot(slot, rk);
    };
    auto key_scales = [&](const half8 (&ka)[KSTEPS], float16v &rk) {
        key_scales_at(ka, rk, reinterpret_cast<float *>(smem + C::SCR_OFF + wave * 128));
    };

    // Softmax numerators of a stream's last tile, the only one that can reach
    // past the chunk end (the tile holding key N, or a tile wholly past the
    // chunk): masked when it does. Every earlier tile of a stream ends before
    // the next tile of the same stream starts, so it lies inside the chunk and
    // takes the unmasked softmax, in a loop body without this branch.
    auto softmax_last = [&](int it, const float16v (&sv)[QT], half8 (&pv_)[QT][2]) {
        const int lim = len - tile_key(it);
        if (lim >= KT)
            softmax<QT, false>(sv, pv_, lsum, 0);
        else
            softmax<QT, true>(sv, pv_, lsum, lim - 4 * h);
    };
    [[maybe_unused]] auto softmax_last_qkn = [&](int it, const float16v (&sv)[QT], const float16v &rkv,
                                                 half8 (&pv_)[QT][2]) {
        const int lim = len - tile_key(it);
        if (lim >= KT)
            softmax_qkn<DT, QT, false>(sv, rkv, rq, pv_, lsum, m_run, real, oacc, 0);
        else
            softmax_qkn<DT, QT, true>(sv, rkv, rq, pv_, lsum, m_run, real, oacc, lim - 4 * h);
    };
    auto load_k = [&](const char *tile, half8 (&a)[KSTEPS]) {
        if constexpr (KM)
            read_k_km<HD>(lds_base(smem, tile + lo.krow), 0, lo.kx, a);
        else
            read_k<HD>(lds_base(smem, tile + lo.k), a);
    };

    if constexpr (C::PRIVATE) {
        // Wave-private ring: buffers ring0 and ring0 + TILE_BYTES.
        const uint32_t ring0 = lds0 + wave * 2 * TILE_BYTES;
        const char *ring = smem + wave * 2 * TILE_BYTES;
        // Q lands before the second tile is issued: at start-up every
        // workgroup's requests reach HBM together, and Q then waits behind
        // less (cold A/B: 3% at (2, 256, 4096), 1% at (64, 8, 8192)).
        issue(0, ring0);
        sync_tile<C::TILE_OPS>();  // this wave's Q share landed; barrier: all of Q landed
        load_q();
        issue(1, ring0 + TILE_BYTES);
        auto step = [&](int it, auto last) {
            wait_vm<C::TILE_OPS>();  // tile it landed (tile it+1 may still be in flight)
            const char *buf = ring + (it & 1) * TILE_BYTES;
            half8 ka[KSTEPS], va[2][DT];
            const char *vbase[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) vbase[dt] = buf + lo.v[dt];
            load_k(buf, ka);
            read_v<HD>(vbase, va);
            wait_lds();              // the buffer is free: refill it with tile it+2
            issue(it + 2, ring0 + (it & 1) * TILE_BYTES);
            float16v s[QT];
            half8 p[QT][2];
            scores<HD, QT>(ka, qf, s);
            if constexpr (QKN) {
                float16v rk;
                key_scales(ka, rk);
                const int lim = len - tile_key(it);
                if (decltype(last)::value && lim < KT)
                    softmax_qkn<DT, QT, true>(s, rk, rq, p, lsum, m_run, real, oacc, lim - 4 * h);
                else
                    softmax_qkn<DT, QT, false>(s, rk, rq, p, lsum, m_run, real, oacc, 0);
            } else if constexpr (decltype(last)::value) {
                softmax_last(it, s, p);
            } else {
                softmax<QT, false>(s, p, lsum, 0);
            }
            pv<HD, QT>(va, p, oacc);
        };
        int it = 0;
        for (; it + 1 < ntiles; ++it) step(it, std::false_type{});
        if (it < ntiles) step(it, std::true_type{});
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
        // Q lands before the tiles after the first are issued (as in the
        // private ring; cold A/B: 1.5% at (16, 256, 4096) and (2, 256, 32768)).
        issue_next();
        // this wave's Q share landed; barrier: all of Q landed
        if constexpr (ONE_ISSUER) {
            if (early)
                sync_tile<T1>();
            else
                sync_tile<0>();
        } else {
            sync_tile<C::TILE_OPS>();
        }
        load_q();                  // done before the first refill overwrites the staging
        for (int j = 1; j < DIST; ++j) issue_next();

        // Unsigned index arithmetic lets the compiler fold each read's constant
        // part into the LDS instruction's offset field.
        auto tile_at = [&](int it) {
            return smem + ((unsigned)it % (unsigned)STAGES) * (unsigned)SB + (unsigned)ks * (unsigned)TILE_BYTES;
        };
        // Step it: tile it landed for every wave, and every wave is done with
        // the buffer that step it refills. The refill itself (issue_next) is
        // issued after the step's MFMAs, so that its scalar descriptor work
        // and DMA issue overlap them instead of delaying the operand reads
        // (cold A/B: 5-6% at (16, 256, 4096) and (2, 256, 32768)).
        auto sync = [&]() {
            sync_tile<(DIST - 1) * C::TILE_OPS>();
        };
        // Two schedules, chosen by the tile shape from cold A/B timings
        // (QT = 1: 64 rows on two query waves; QT = 2: 128 and 256 rows).
        if constexpr (QT == 1) {
            // Two-stage pipeline with a phase offset. Step `it` runs the first
            // product of tile it, the second product of tile it-1 and one
            // softmax: of tile it in an early wave (after its first product,
            // beside its second), of tile it-1 in a late wave (before both
            // products). The two waves of a SIMD are one early
            // (w < NWAVES/2) and one late (w + NWAVES/2): the barrier of each
            // step starts both together, and then one issues MFMAs while the
            // other issues VALU. The early wave, the stream's first query
            // wave, also issues the stream's DMA.
            float16v s[QT];
            half8 p[QT][2];
            [[maybe_unused]] float16v rk;  // QK normalisation: the key scales of the tile in s
            // QK normalisation: the early wave computes each tile's key scales
            // into its stream's slot (two per stream, by tile parity); the
            // late wave, which takes tile it's softmax one step later, reads
            // them from there.
            [[maybe_unused]] auto kslot = [&](int it) {
                return reinterpret_cast<float *>(smem + C::SCR_OFF + (ks * 2 + (it & 1)) * 128);
            };
            auto g1 = [&](int it) {
                half8 a[KSTEPS];
                load_k(tile_at(it), a);
                scores<HD, QT>(a, qf, s);
                if constexpr (QKN)
                    if (early) key_scales_at(a, rk, kslot(it));
            };
            // Tiles before a stream's last (it <= niter - 2) lie inside the chunk.
            // With QK normalisation the softmax may rescale W and L: in either
            // phase order it runs before the tile's own second product, so
            // W and L then hold only tiles already relative to the old maximum.
            auto sm = [&]() {
                if constexpr (QKN)
                    softmax_qkn<DT, QT, false>(s, rk, rq, p, lsum, m_run, real, oacc, 0);
                else
                    softmax<QT, false>(s, p, lsum, 0);
            };
            auto g2 = [&](int it) {
                half8 a[2][DT];
                const char *vbase[DT];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) vbase[dt] = lds_base(smem, tile_at(it) + lo.v[dt]);
                read_v<HD>(vbase, a);
                pv<HD, QT>(a, p, oacc);
            };
            const int niter = ntiles;
            // Step it needs the K part of tile it and the V part of tile
            // it-1, which was issued before it: the early wave's wait leaves
            // the V part of tile it in flight (it issues a tile's K
            // instructions before its V instructions and they complete in
            // order); the late wave issues no DMA and waits only at the
            // barrier, which makes the tile visible to it.
            auto sync = [&]() {
                if (early)
                    sync_tile<(DIST - 1) * T1 + T1 / 2>();
                else
                    sync_tile<0>();
            };
            // The scheduling barriers keep the compiler from merging the
            // phases. The orders run in separate loops, so that neither one's
            // live values burden the other's registers.
            if (wave >= C::NWAVES / 2) {  // late
                sync();                   // step 0
                g1(0);
                issue_next();
                for (int it = 1; it < niter; ++it) {
                    sync();
                    if constexpr (QKN) scales_from_slot(kslot(it - 1), rk);
                    sm();                 // tile it-1
                    __builtin_amdgcn_sched_barrier(0);
                    g1(it);
                    g2(it - 1);
                    issue_next();
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {                      // early
                // The second product of tile it-1 and the softmax of tile it
                // share one scheduling region (one P buffer: the softmax's
                // conversions into P wait for the MFMAs that read it).
                sync();                   // step 0
                g1(0);
                issue_next();
                int it = 1;
                if (niter > 1) {
                    sm();
                    for (; it + 1 < niter; ++it) {
                        sync();
                        g1(it);
                        issue_next();
                        __builtin_amdgcn_sched_barrier(0);
                        g2(it - 1);
                        sm();             // tile it
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    sync();               // step niter-1: the last tile's softmax may be masked
                    g1(it);
                    issue_next();
                    __builtin_amdgcn_sched_barrier(0);
                    g2(it - 1);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // The late wave reads the last tile's key scales after the
            // barrier below: the early wave writes them in its last step.
            if constexpr (QKN) {
                if (early) softmax_last_qkn(niter - 1, s, rk, p);
            } else {
                softmax_last(niter - 1, s, p);
            }
            if (early)  // the V part of the last tile landed for every wave
                sync_tile<DIST * T1>();
            else
                sync_tile<0>();
            if constexpr (QKN) {
                if (!early) {
                    scales_from_slot(kslot(niter - 1), rk);
                    softmax_last_qkn(niter - 1, s, rk, p);
                }
            }
            g2(niter - 1);
        } else {
            // Two-stage pipeline, the same order in every wave. Step `it`
            // reads tile it's K operand and runs the first product of tile it;
            // then the second product of tile it-1 (its V operand read in the
            // previous step) and the softmax of tile it go out together, so
            // that the wave's own VALU work overlaps its second-product MFMAs
            // (one P buffer: the softmax's conversions into P wait for the
            // MFMAs that read it, its exps need not); last, it reads tile
            // it's V operand. Every wave is done with tile it-2 after step
            // it-1, which frees its buffer for the refill at step it.
            float16v s[QT];
            half8 p[QT][2];
            half8 ka[KSTEPS], va[2][DT];
            auto rk = [&](int it) { load_k(tile_at(it), ka); };
            auto rv = [&](int it) {
                const char *vbase[DT];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) vbase[dt] = lds_base(smem, tile_at(it) + lo.v[dt]);
                read_v<HD>(vbase, va);
            };
            auto mm1 = [&]() { scores<HD, QT>(ka, qf, s); };
            auto mm2 = [&]() { pv<HD, QT>(va, p, oacc); };
            // Tiles before a stream's last (it <= niter - 2) lie inside the chunk.
            auto sm = [&]() { softmax<QT, false>(s, p, lsum, 0); };
            const int niter = ntiles;
            // The scheduling barriers keep the steps' phases in this order.
            sync();             // step 0
            rk(0);
            mm1();
            issue_next();
            __builtin_amdgcn_sched_barrier(0);
            rv(0);
            int it = 1;
            if (niter > 1) {
                sm();
                for (; it + 1 < niter; ++it) {
                    sync();
                    rk(it);
                    mm1();
                    issue_next();
                    __builtin_amdgcn_sched_barrier(0);
                    mm2();      // tile it-1
                    sm();       // tile it
                    __builtin_amdgcn_sched_barrier(0);
                    rv(it);
                    __builtin_amdgcn_sched_barrier(0);
                }
                sync();         // step niter-1: the last tile's softmax may be masked
                rk(it);
                mm1();
                issue_next();
                __builtin_amdgcn_sched_barrier(0);
                mm2();
                __builtin_amdgcn_sched_barrier(0);
                rv(it);
            }
            softmax_last(niter - 1, s, p);
            mm2();
        }
        sync_tile<0>();  // no DMA in flight, every wave done with the ring
    }

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
            const float lfull = mine + __shfl_xor(mine, 32);
            if (h == 0) lreg[qr] = lfull;
            if constexpr (QKN)  // a stream with no key in the row has no reference: -inf
                if (h == 0) lreg[32 * QT + qr] = real[qt] ? m_run[qt] : -__builtin_inff();
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
        // QK normalisation: the streams' W and L are relative to their own
        // reference maxima; bring them to the largest, mstar, first.
        [[maybe_unused]] float mstar = -__builtin_inff();
        if constexpr (QKN) {
#pragma unroll
            for (int s2 = 0; s2 < KS; ++s2) {
                const float *lreg = (const float *)(smem + (qw * KS + s2) * C::RED_BYTES + 32 * QT * G::RED_ROW_BYTES);
                mstar = __builtin_fmaxf(mstar, lreg[32 * QT + qr]);
            }
        }
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            const char *reg = smem + (qw * KS + s2) * C::RED_BYTES;
            const float *lreg = (const float *)(reg + 32 * QT * G::RED_ROW_BYTES);
            if constexpr (QKN) {
                const float ms = lreg[32 * QT + qr];
                const float f = ms > -__builtin_inff() ? __builtin_amdgcn_exp2f(ms - mstar) : 0.f;
#pragma unroll
                for (int x = 0; x < C::VPL; x += 4) {
                    const float4v t = *(const float4v *)(reg + qr * G::RED_ROW_BYTES + (d0 + x) * 4);
#pragma unroll
                    for (int y = 0; y < 4; ++y) acc[x + y] = __builtin_fmaf(f, t[y], acc[x + y]);
                }
                l = __builtin_fmaf(f, lreg[qr], l);
            } else {
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
        }
        const int row = qbase + qr;
        if (row < M) {
            if (nsplit == 1) {
                _Float16 *dst = o + b * st.o_b + (size_t)row * st.o_i + d0;
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
                // With QK normalisation W_s, L_s are relative to 2^mstar, so the
                // workspace gets lse_s = mstar + log2(L_s) instead of L_s.
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
                if (ks == 0 && d0 == 0) {
                    if constexpr (QKN)
                        ws_l[prow] = mstar + __builtin_log2f(l);
                    else
                        ws_l[prow] = l;
                }
            }
        }
    }
}

// Combine: HD/4 threads per output row, 4 head dims each.
// O = fp16(sum_s L_s o_s / sum_s L_s), both sums in split order (from 32
// splits, the grouped form below sums four quarters, then the quarters).
// With LSE (QK normalisation) the workspace holds lse_s = log2 of each
// split's weight mass; the weights are then 2^(lse_s - max_s lse_s).
// The partials sit in L2 or the Infinity Cache and each thread is bound by
// their latency. Up to four splits, a thread issues every load before it sums
// any; more splits go through an 8-way unrolled loop (each form measured the
// faster one in its range on MI355X). Both sum in split order.
template <int HD, bool LSE>
__global__ __launch_bounds__(256) void gqa_combine_kernel(const _Float16 *__restrict__ ws_o,
                                                          const float *__restrict__ ws_l,
                                                          _Float16 *__restrict__ o, long long o_b, int o_i,
                                                          int M, long long rows, int nsplit) {
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long row = gid / (HD / 4);
    const int c = (int)(gid % (HD / 4));
    if (row >= rows) return;
    float l = 0.f;
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    [[maybe_unused]] float lmax = -__builtin_inff();
    if constexpr (LSE)
        for (int s = 0; s < nsplit; ++s) lmax = __builtin_fmaxf(lmax, ws_l[(long long)s * rows + row]);
    auto weight = [&](float ls) {
        if constexpr (LSE) return ls > -__builtin_inff() ? __builtin_amdgcn_exp2f(ls - lmax) : 0.f;
        return ls;
    };
    if (nsplit <= 4) {
        float ls[4];
        half4 os[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < nsplit) {
                const long long prow = (long long)s * rows + row;
                ls[s] = ws_l[prow];
                os[s] = *reinterpret_cast<const half4 *>(ws_o + prow * HD + 4 * c);
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < nsplit) {
                const float w = weight(ls[s]);
                l += w;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += w * (float)os[s][i];
            }
        }
    } else {
#pragma unroll 8
        for (int s = 0; s < nsplit; ++s) {
            const long long prow = (long long)s * rows + row;
            const float w = weight(ws_l[prow]);
            const half4 os = *reinterpret_cast<const half4 *>(ws_o + prow * HD + 4 * c);
            l += w;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += w * (float)os[i];
        }
    }
    half4 hv;
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = (_Float16)(acc[i] / l);
    const long long b = row / M;
    *reinterpret_cast<half4 *>(o + b * o_b + (row - b * M) * o_i + 4 * c) = hv;
}

// Combine over many splits: few rows (a long key range on a
// small batch) leave the one-thread-per-4-columns form with few workgroups,
// each walking every split in turn. Here four groups of 64 threads share the
// same rows: group g sums the g-th contiguous quarter of the splits in split
// order, and group 0 then adds groups 1, 2, 3 in that order (fixed, so the
// result is deterministic) before the division. With LSE every group first
// takes the maximum lse over its quarter; the four maxima meet in LDS, so the
// weights 2^(lse_s - max) use the same maximum as the one-group form.
template <int HD, bool LSE>
__global__ __launch_bounds__(256) void gqa_combine_grouped_kernel(const _Float16 *__restrict__ ws_o,
                                                                  const float *__restrict__ ws_l,
                                                                  _Float16 *__restrict__ o, long long o_b,
                                                                  int o_i, int M, long long rows, int nsplit) {
    constexpr int CPR = HD / 4;    // threads per row, 4 head dims each
    constexpr int RPB = 64 / CPR;  // rows per workgroup
    __shared__ float red[3][5][64];
    [[maybe_unused]] __shared__ float gmax[4][64];
    const int g = threadIdx.x >> 6, t = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * RPB + t / CPR;
    const int c = t % CPR;
    const bool valid = row < rows;
    const int s0 = g * nsplit / 4, s1 = (g + 1) * nsplit / 4;
    [[maybe_unused]] float lmax = -__builtin_inff();
    if constexpr (LSE) {
        if (valid)
            for (int s = s0; s < s1; ++s) lmax = __builtin_fmaxf(lmax, ws_l[(long long)s * rows + row]);
        gmax[g][t] = lmax;
        __syncthreads();
        lmax = __builtin_fmaxf(__builtin_fmaxf(gmax[0][t], gmax[1][t]), __builtin_fmaxf(gmax[2][t], gmax[3][t]));
    }
    float l = 0.f;
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    if (valid) {
#pragma unroll 8
        for (int s = s0; s < s1; ++s) {
            const long long prow = (long long)s * rows + row;
            float w = ws_l[prow];
            if constexpr (LSE) w = w > -__builtin_inff() ? __builtin_amdgcn_exp2f(w - lmax) : 0.f;
            const half4 os = *reinterpret_cast<const half4 *>(ws_o + prow * HD + 4 * c);
            l += w;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += w * (float)os[i];
        }
    }
    if (g > 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) red[g - 1][i][t] = acc[i];
        red[g - 1][4][t] = l;
    }
    __syncthreads();
    if (g == 0 && valid) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            l += red[j][4][t];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] += red[j][i][t];
        }
        half4 hv;
#pragma unroll
        for (int i = 0; i < 4; ++i) hv[i] = (_Float16)(acc[i] / l);
        const long long b = row / M;
        *reinterpret_cast<half4 *>(o + b * o_b + (row - b * M) * o_i + 4 * c) = hv;
    }
}

// K repack for contiguous head-dim-major K whose rows (N keys) are not
// 16-byte aligned: each thread writes 8 keys of one row of the copy, rows of
// ceil8(N) keys, zero past N.
__global__ __launch_bounds__(256) void repack_k_kernel(const _Float16 *__restrict__ src,
                                                       _Float16 *__restrict__ dst, long long rows, int N,
                                                       int n8) {
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const int per_row = n8 / 8;
    const long long row = gid / per_row;
    const int c = (int)(gid - row * per_row) * 8;
    if (row >= rows) return;
    const _Float16 *s = src + row * N;
    half8 out;
#pragma unroll
    for (int j = 0; j < 8; ++j) out[j] = c + j < N ? s[c + j] : (_Float16)0.f;
    *reinterpret_cast<half8 *>(dst + row * n8 + c) = out;
}

// Enqueues `kernel` on `stream` and returns the status of this launch alone
// (hipLaunchKernel's own result), not an error an earlier HIP call of the
// caller may have left pending.
template <typename... P, typename... A>
int launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream, A &&...args) {
    static_assert(sizeof...(P) == sizeof...(A), "argument count");
    std::tuple<P...> vals(std::forward<A>(args)...);  // the kernel's own parameter types
    void *ptrs[sizeof...(P)];
    std::apply([&](auto &...v) {
        int i = 0;
        ((ptrs[i++] = static_cast<void *>(&v)), ...);
    }, vals);
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs, 0, stream);
}

template <int HD, int QT, int QW, int KS, bool KM, bool QKN>
int launch_partial_layout(const mga::Plan &p, const _Float16 *q, const _Float16 *k, const _Float16 *v,
                          _Float16 *o, _Float16 *w, float *l, hipStream_t st) {
    static_assert(32 * QT * QW == 32 || 32 * QT * QW == 64 || 32 * QT * QW == 128 || 32 * QT * QW == 256,
                  "rows per workgroup");
    const int pairs = p.B * p.splits;
    const int groups = (pairs + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * p.mtiles));
    return launch(gqa_partial_kernel<HD, QT, QW, KS, KM, QKN>, grid, dim3(64 * QW * KS), st, q, k, v, o, w, l,
                  p.st, p.B, p.M, p.N, p.chunk_keys, p.splits, p.mtiles, p.eps);
}

template <int HD, int QT, int QW, int KS, bool QKN = false>
int launch_partial_cfg(const mga::Plan &p, const _Float16 *q, const _Float16 *k, const _Float16 *v,
                       _Float16 *o, _Float16 *w, float *l, hipStream_t st) {
    if (p.key_major) return launch_partial_layout<HD, QT, QW, KS, true, QKN>(p, q, k, v, o, w, l, st);
    return launch_partial_layout<HD, QT, QW, KS, false, QKN>(p, q, k, v, o, w, l, st);
}

}  // namespace

// Library-owned device scratch of mga_gqa_forward_noalloc (the workspace of
// callers that cannot allocate): kScratchBytes per GPU, allocated with the
// code object when the library is first used on that GPU and held until the
// process ends. Host code never names it directly: scratch_ptr returns the
// address the runtime reports for the current device.
static __device__ __align__(256) char scratch[mga::kScratchBytes];

namespace mga {

int scratch_ptr(void **out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *per_device[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));  // with `dev` current
        if (e != hipSuccess) return (int)e;
        if (!ptr) return (int)hipErrorInvalidSymbol;
        per_device[dev] = ptr;
    }
    *out = per_device[dev];
    return 0;
}

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
    if (p.qknorm) {
        switch (p.variant) {
        // 32 rows on 4 waves (two workgroups per CU) and head dim 128 on 2
        // waves, as in the plain path: cold A/B against 8 and 4 waves,
        // (64, 8, 8192) 32.00 -> 30.80 us (4 -> 8 splits), (64, 1, 4096, 128)
        // 32.81 -> 30.18, (16, 1, 16384, 128) 34.66 -> 32.24.
        case kVariantDecode: return launch_partial_cfg<64, 1, 1, 4, true>(p, qh, kh, vh, oh, w, l, st);
        case kVariantSmall: return launch_partial_cfg<64, 2, 1, 8, true>(p, qh, kh, vh, oh, w, l, st);
        case kVariantSmallShared: return launch_partial_cfg<64, 1, 2, 4, true>(p, qh, kh, vh, oh, w, l, st);
        case kVariantDecode128: return launch_partial_cfg<128, 1, 1, 2, true>(p, qh, kh, vh, oh, w, l, st);
        default: return (int)hipErrorInvalidValue;
        }
    }
    switch (p.variant) {
    // 32 rows on 4 waves (two workgroups per CU): cold A/B against 8 waves at
    // 4 splits, (64, 8, 8192) 30.05 -> 28.17 us at 8 splits, (2, 256, 4096)
    // 8.45 -> 7.57 us.
    case kVariantDecode: return launch_partial_cfg<64, 1, 1, 4>(p, qh, kh, vh, oh, w, l, st);
    case kVariantSmall: return launch_partial_cfg<64, 2, 1, 8>(p, qh, kh, vh, oh, w, l, st);
    case kVariantMedium: return launch_partial_cfg<64, 2, 2, 4>(p, qh, kh, vh, oh, w, l, st);
    case kVariantLarge: return launch_partial_cfg<64, 2, 4, 2>(p, qh, kh, vh, oh, w, l, st);
    case kVariantSmallShared: return launch_partial_cfg<64, 1, 2, 4>(p, qh, kh, vh, oh, w, l, st);
    // Head dim 128 on 2 waves (one workgroup per CU at the policy's splits,
    // each wave streaming twice the tiles): cold A/B against 4 waves,
    // (64, 1, 4096) 29.65 -> 28.3 us, (16, 1, 16384) 30.76 -> 29.26,
    // (64, 32, 4096) 30.00 -> 28.85.
    case kVariantDecode128: return launch_partial_cfg<128, 1, 1, 2>(p, qh, kh, vh, oh, w, l, st);
    default: return (int)hipErrorInvalidValue;
    }
}

int launch_repack(const Plan &p, const void *k, void *ws, void *stream) {
    const int n8 = (p.N + 7) & ~7;
    const long long rows = (long long)p.B * p.D;
    const long long threads = rows * (n8 / 8);
    const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
    return launch(repack_k_kernel, grid, dim3(kThreads), (hipStream_t)stream, (const _Float16 *)k,
                  (_Float16 *)((char *)ws + p.repack_off), rows, p.N, n8);
}

int launch_combine(const Plan &p, void *o, const void *ws, void *stream) {
    _Float16 *w = nullptr;
    float *l = nullptr;
    ws_split(p, ws, &w, &l);
    const long long rows = (long long)p.B * p.M;
    hipStream_t st = (hipStream_t)stream;
    _Float16 *oh = (_Float16 *)o;
    if (p.splits >= kGroupedCombineSplits) {
        const long long rpb = 64 / (p.D / 4);
        const dim3 ggrid((unsigned)((rows + rpb - 1) / rpb));
        auto kern = p.D == 128 ? (p.qknorm ? gqa_combine_grouped_kernel<128, true> : gqa_combine_grouped_kernel<128, false>)
                               : (p.qknorm ? gqa_combine_grouped_kernel<64, true> : gqa_combine_grouped_kernel<64, false>);
        return launch(kern, ggrid, dim3(kThreads), st, w, l, oh, p.st.o_b, p.st.o_i, p.M, rows, p.splits);
    }
    const long long threads = rows * (p.D / 4);
    const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
    auto kern = p.D == 128 ? (p.qknorm ? gqa_combine_kernel<128, true> : gqa_combine_kernel<128, false>)
                           : (p.qknorm ? gqa_combine_kernel<64, true> : gqa_combine_kernel<64, false>);
    return launch(kern, grid, dim3(kThreads), st, w, l, oh, p.st.o_b, p.st.o_i, p.M, rows, p.splits);
}

}  // namespace mga
