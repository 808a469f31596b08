// Split-KV partial kernel and combine kernel for the GQA exp-sum-div graph on
// gfx950 (MI355X, CDNA4).
//
// Graph (Mirage GQA tutorial, "Mirage: Define GQA Computation Graph"):
//   A = Q K, E = exp(A), S = rowsum(E), O = (E / S) V   -- no scale, no max.
// Split-KV form (kaispace blog, sections 2.1 and 4.2-4.3: a for-loop over the
// key dimension that accumulates, then a combine block graph): a workgroup
// owns (batch row b, query tile, key chunk) and accumulates
//   W = sum_n fp16(e_n) V[n]   and   L = sum_n e_n
// over its chunk; O = sum_s W_s / sum_s L_s. With no running maximum the
// partials combine by plain sums.
//
// Partial kernel. A workgroup has QW x KS waves: QW query groups of 32*QT
// rows each, times KS key streams. Stream ks takes every KS-th 32-key tile of
// the chunk; its QW waves share that tile through LDS. Per tile and wave:
//   * S^T = K^T Q^T on v_mfma_f32_32x32x16_f16: keys on the accumulator rows,
//     queries on its columns; Q^T stays in registers for the whole kernel.
//   * E = exp2(S') in fp32, where S' = (log2(e) Q) K comes from Q pre-scaled
//     once per workgroup; L += E (fp32 adds); P = fp16(E) (nearest even). In the 32x32 accumulator layout a lane holds 16 keys of one
//     query, in exactly the order the next MFMA's B operand needs (two 16-key
//     k-steps, 8 consecutive accumulator registers each), so the scores never
//     leave registers.
//   * O^T += V^T P^T on the same MFMA.
// K (head-dim-major) and V (key-major) are copied HBM -> LDS as they are laid
// out in memory, by buffer_load ... lds (no registers involved), into a ring
// of 4 buffers (two tiles per stream in flight ahead of the pair being
// computed). The MFMA operands need the contraction index along each lane's
// 8 values, which is the slow index of both tiles; ds_read_b64_tr_b16
// delivers that transpose: within each group of 16 lanes it returns
// result[i][j] = source[4j + i/4][i % 4] over the 16 lanes' 4-element reads,
// i.e. lane i receives column i of a 4 x 16 block. LDS rows are XOR-swizzled
// at 32-byte granularity so that the four rows of such a block fall in
// distinct banks.
// After the loop the KS streams of a query group are summed in LDS in a fixed
// order; with one split the kernel writes O = fp16(W / L), otherwise W and L
// go to the caller's workspace for the combine kernel.
//
// Bounds. Every K/V access goes through a buffer descriptor that covers only
// batch b's K (or V) array: keys past N read as zero (V) or as other keys of
// the same batch (K, whose rows continue in memory); either way the scores of
// keys past the chunk end are forced to E = 0. Tiles wholly past the chunk
// end are issued with an offset past the descriptor's end, so they move no
// data and write zeros. Query rows past M are zero-filled and never stored.

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

constexpr int HD = mga::kHeadDim;            // 64
constexpr int KT = 32;                       // keys per tile
constexpr int TILE_BYTES = KT * HD * 2 * 2;  // K part 4 KiB + V part 4 KiB
constexpr int K_ROW_BYTES = KT * 2;          // 64
constexpr int V_ROW_BYTES = HD * 2;          // 128
constexpr int V_PART = KT * HD * 2;          // byte offset of the V part in a tile
constexpr int RED_ROW_BYTES = HD * 4 + 16;   // fp32 row of 64 + 16-byte pad (bank spread)
constexpr float LOG2E = 1.4426950408889634f;
constexpr int BUFFER_FLAGS = 0x00020000;     // gfx9 raw buffer descriptor, dword 3

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
// V part: [32 keys][64 d] fp16, 128-byte rows of four 32-byte units; the unit
// index is XORed with the row's low two bits.
__device__ __forceinline__ int v_off(int key, int col_byte) {
    return V_PART + key * V_ROW_BYTES + (((col_byte >> 5) ^ (key & 3)) << 5) + (col_byte & 31);
}

template <int QT, int QW, int KS>
struct Partial {
    static constexpr int NWAVES = QW * KS;
    static constexpr int ROWS = 32 * QT * QW;  // query rows per workgroup
    static_assert(4 % QW == 0, "QW must divide the 4 K and 4 V DMA instructions of a tile");
    static constexpr int PER = 4 / QW;         // K (and V) DMA instructions per wave per tile
    // LDS ring: each buffer holds one tile per stream. Step `it` reads tile it
    // only, so after its barrier the buffer of tile it-1 is free and is
    // refilled with tile it+STAGES-1: STAGES-1 tiles are in flight.
    static constexpr int STAGE_BYTES = KS * TILE_BYTES;
    static constexpr int RED_BYTES = 32 * QT * RED_ROW_BYTES + 32 * QT * 4;  // one wave's epilogue region
    static constexpr int STAGES = (160 * 1024) / STAGE_BYTES < 10 ? (160 * 1024) / STAGE_BYTES : 10;
    // With 4 or fewer streams the ring is deep enough for the three-phase
    // software pipeline (a step reads tiles it and it-2 and keeps it-1, so it
    // refills tile it-3's buffer); with 8 streams each step handles one tile
    // and refills the buffer of tile it-1.
    static constexpr bool PIPE = STAGES >= 5;
    static constexpr int DIST = PIPE ? STAGES - 3 : STAGES - 1;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES > NWAVES * RED_BYTES ? STAGES * STAGE_BYTES
                                                                              : NWAVES * RED_BYTES;
    static_assert(STAGES >= 2, "ring depth");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert((DIST - 1) * 2 * PER < 64, "vmcnt range");
    static constexpr int DW = HD / KS;                // head dims each wave finalises
    static constexpr int VPL = 32 * QT * DW / 64;     // values per lane in the final write
    static_assert(KS == 1 || (VPL >= 4 && VPL % 4 == 0), "final write granularity");
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
// across them; completion is waited for explicitly (sync_tile).
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding, then meet the other waves at the workgroup barrier.
template <int N>
__device__ __forceinline__ void sync_tile() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "n"(N) : "memory");
}

// Issue this wave's DMA share of one stream's tile (keys ts .. ts+31) into
// the LDS tile at byte address `lds`. A tile is 8 instructions of 64 lanes x
// 16 bytes: 4 fill the K part (16 rows of 64 bytes each), 4 the V part (8 rows
// of 128 bytes each); each of the QW waves sharing the tile issues 4/QW of
// each. Key chunks at or past N, and whole tiles at or past the chunk end,
// are given an offset past the descriptor and read zero.
template <int QW>
__device__ __forceinline__ void issue_tile(i32x4 krsrc, i32x4 vrsrc, uint32_t lds, int N, int ts,
                                           int kend, int qw, int lane) {
    constexpr int PER = 4 / QW;
    const bool live = ts < kend;
    const uint32_t oob = (uint32_t)N * (HD * 2);
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const int r = qw * PER + x;  // K rows 16r .. 16r+15
        const uint32_t d = 16 * r + (lane >> 2);
        const uint32_t lc = (lane & 3) ^ (((d >> 1) & 1) << 1);
        const uint32_t key = (uint32_t)ts + 8 * lc;
        const uint32_t off = live && key < (uint32_t)N ? (d * (uint32_t)N + key) * 2 : oob;
        dma16(krsrc, off, lds + r * 1024);
    }
#pragma unroll
    for (int x = 0; x < PER; ++x) {
        const int r = qw * PER + x;  // V rows 8r .. 8r+7
        const uint32_t kr = 8 * r + (lane >> 3);
        const uint32_t lc = (lane & 7) ^ ((kr & 3) << 1);
        const uint32_t off = live ? (((uint32_t)ts + kr) * HD + 8 * lc) * 2 : oob;
        dma16(vrsrc, off, lds + V_PART + r * 1024);
    }
}

// Per-lane LDS byte offsets (within a tile) of the transposed operand reads.
// The K part's swizzle depends on bit 1 of the row, which the +4 and +16 row
// steps leave unchanged, and the V part's on the row's low two bits, which
// the +8 and +16 row steps leave unchanged; so one base per read family
// plus immediate offsets covers every read.
struct LaneOffsets {
    int k;      // K part, head dims 8h+jr (+4, +16 kk), keys 16 g1 + 4c
    int v[2];   // V part, keys 4h+jr (+8, +16 t), head dims 32 dt + 16 g1 + 4c
};
__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
    const int h = lane >> 5, g1 = (lane >> 4) & 1, jr = (lane & 15) >> 2, cb = 8 * (lane & 3);
    LaneOffsets r;
    r.k = k_off(8 * h + jr, 32 * g1 + cb);
    r.v[0] = v_off(4 * h + jr, 32 * g1 + cb);
    r.v[1] = v_off(4 * h + jr, 64 + 32 * g1 + cb);
    return r;
}

// First product of one tile for one wave (32*QT queries): S^T = K^T Q^T.
template <int QT>
__device__ __forceinline__ void tile_scores(const char *kb, const half8 (&qf)[QT][4],
                                            float16v (&s)[QT]) {
    half8 a[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        a[kk] = cat8(tr_read(kb + kk * 16 * K_ROW_BYTES), tr_read(kb + kk * 16 * K_ROW_BYTES + 4 * K_ROW_BYTES));
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        s[qt] = float16v{};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            s[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[kk], qf[qt][kk], s[qt], 0, 0, 0);
    }
}

// Softmax numerators of one tile: E = exp2(S) (scores are in log2 units),
// L += E, P = fp16(E) rounded to nearest. In the 32x32 accumulator layout
// register r of lane l holds key 8*(r/4) + 4*(l/32) + r%4 of query l%32, so
// registers 8t..8t+7 are exactly the 8 k-slots of the second product's
// B operand for keys 16t..16t+15.
template <int QT>
__device__ __forceinline__ void tile_softmax(const float16v (&s)[QT], half8 (&p)[QT][2],
                                             float (&lsum)[QT]) {
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(s[qt][r]);
        float a0 = 0.f, a1 = 0.f;  // two short chains instead of one long one
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            a0 += e[r];
            a1 += e[r + 1];
        }
        lsum[qt] += a0 + a1;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const half2v hv = __builtin_convertvector(float2v{e[8 * t + 2 * j], e[8 * t + 2 * j + 1]}, half2v);
                p[qt][t][2 * j] = hv[0];
                p[qt][t][2 * j + 1] = hv[1];
            }
        }
    }
}

// Second product of one tile: O^T += V^T P^T.
template <int QT>
__device__ __forceinline__ void tile_pv(const char *vb0, const char *vb1, const half8 (&p)[QT][2],
                                        float16v (&oacc)[2][QT]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
            const char *vb = (dt == 0 ? vb0 : vb1) + t * 16 * V_ROW_BYTES;
            const half8 a = cat8(tr_read(vb), tr_read(vb + 8 * V_ROW_BYTES));
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
                oacc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, p[qt][t], oacc[dt][qt], 0, 0, 0);
        }
    }
}

template <int QT, int QW, int KS>
__global__ __launch_bounds__(64 * QW * KS) void gqa_partial_kernel(
    const _Float16 *__restrict__ q, const _Float16 *__restrict__ k,
    const _Float16 *__restrict__ v, _Float16 *__restrict__ o, float *__restrict__ ws_w,
    float *__restrict__ ws_l, int B, int M, int N, int chunk_keys, int nsplit, int mtiles) {
    using C = Partial<QT, QW, KS>;
    constexpr int STAGES = C::STAGES, DIST = C::DIST, SB = C::STAGE_BYTES;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

    // Workgroup -> (batch, split, query tile). Consecutive workgroup ids go to
    // different XCDs (id % 8); the query tiles of one (batch, split) pair get
    // ids 8 apart so they run on the same XCD and share its L2 copy of K/V.
    const int wid = blockIdx.x;
    const int pair = (wid / (8 * mtiles)) * 8 + (wid & 7);
    const int mtile = (wid >> 3) % mtiles;
    if (pair >= B * nsplit) return;
    const int b = pair / nsplit, split = pair - b * nsplit;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int qw = wave / KS, ks = wave - qw * KS;
    const int h = lane >> 5;

    const int kstart = split * chunk_keys;
    const int kend = min(N, kstart + chunk_keys);
    const int niter = (kend - kstart + KS * KT - 1) / (KS * KT);

    const int qbase = mtile * C::ROWS + qw * 32 * QT;  // first query row of this wave

    const i32x4 krsrc = make_rsrc(k + (size_t)b * HD * N, (uint32_t)N * HD * 2);
    const i32x4 vrsrc = make_rsrc(v + (size_t)b * N * HD, (uint32_t)N * HD * 2);
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)(smem));
    const LaneOffsets lo = lane_offsets(lane);

    // Pre-loop: Q^T fragments (B operand). Lane holds query qbase + 32*qt +
    // (lane & 31), head dims 16*kk + 8*h .. +7, pre-scaled by log2(e) (fp32
    // product rounded to fp16) so that the first product yields log2-domain
    // scores and E = exp2(S) needs no per-score multiply.
    half8 qf[QT][4];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int row = qbase + 32 * qt + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            half8 x = row < M ? *reinterpret_cast<const half8 *>(q + ((size_t)b * M + row) * HD + 16 * kk + 8 * h)
                              : half8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = (_Float16)((float)x[j] * LOG2E);
            qf[qt][kk] = x;
        }
    }

    float16v oacc[2][QT];
    float lsum[QT];  // per lane: its 16 keys of every tile
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        oacc[0][qt] = float16v{};
        oacc[1][qt] = float16v{};
        lsum[qt] = 0.f;
    }

    auto tile_start = [&](int it) { return kstart + (it * KS + ks) * KT; };
    // Tiles are issued in order; buffer (it % STAGES) holds tile it.
    int fill_buf = 0;   // buffer receiving the next issued tile
    int fill_it = 0;    // next tile to issue
    auto issue_next = [&]() {
        issue_tile<QW>(krsrc, vrsrc, lds0 + fill_buf * SB + ks * TILE_BYTES, N, tile_start(fill_it), kend,
                       qw, lane);
        fill_buf = fill_buf + 1 == STAGES ? 0 : fill_buf + 1;
        ++fill_it;
    };
    for (int j = 0; j < DIST; ++j) issue_next();

    // Keys at or past the chunk end were loaded as zero K columns and zero V
    // rows: their S is 0, their E exactly 1 and their O contribution nothing;
    // they are removed from L by count at the end.
    float masked = 0.f;
    auto count_masked = [&](int it) { masked += (float)min(KT, max(0, tile_start(it) + KT - kend)); };
    auto tile_at = [&](int it) { return smem + (it % STAGES) * SB + ks * TILE_BYTES; };
    auto sync = [&]() {
        sync_tile<(DIST - 1) * 2 * C::PER>();  // tile it landed for every wave; its refill target is free
        issue_next();
    };
    if constexpr (C::PIPE) {
        // Step `it` runs the first product of tile it, the softmax numerators
        // of tile it-1 and the second product of tile it-2. The three are
        // independent, so each wave's instruction stream always holds both
        // MFMA and VALU work. The second product runs first in a step, so the
        // softmax of the same step may overwrite the weights p it consumed;
        // the scores alternate between s0 and s1.
        float16v s0[QT], s1[QT];
        half8 p[QT][2];
        auto g1 = [&](int it, float16v (&sv)[QT]) { tile_scores<QT>(tile_at(it) + lo.k, qf, sv); };
        auto sm = [&](int it, const float16v (&sv)[QT]) {
            tile_softmax<QT>(sv, p, lsum);
            count_masked(it);
        };
        auto g2 = [&](int it) { tile_pv<QT>(tile_at(it) + lo.v[0], tile_at(it) + lo.v[1], p, oacc); };

        sync();                 // step 0
        g1(0, s0);
        sync();                 // step 1 (tile 1 may lie past the chunk: zeros, unused)
        g1(1, s1);
        sm(0, s0);
        int it = 2;
        for (; it + 1 < niter; it += 2) {
            sync();
            g2(it - 2);
            g1(it, s0);
            sm(it - 1, s1);
            sync();
            g2(it - 1);
            g1(it + 1, s1);
            sm(it, s0);
        }
        if (it < niter) {       // one more full step, it even
            sync();
            g2(it - 2);
            g1(it, s0);
            sm(it - 1, s1);
            ++it;
        }
        // Drain: tiles niter-2 and niter-1 still need their second product,
        // tile niter-1 its softmax (niter == 1: only tile 0's product).
        if (niter == 1) {
            g2(0);
        } else if (it & 1) {    // last step even: tile niter-1's scores in s0
            g2(niter - 2);
            sm(niter - 1, s0);
            g2(niter - 1);
        } else {                // last step odd: tile niter-1's scores in s1
            g2(niter - 2);
            sm(niter - 1, s1);
            g2(niter - 1);
        }
    } else {
        int cur = 0;  // buffer of tile it
        for (int it = 0; it < niter; ++it) {
            sync();   // tile it landed for every wave; tile it-1's buffer is free
            const char *tile = smem + cur * SB + ks * TILE_BYTES;
            float16v s[QT];
            half8 p[QT][2];
            tile_scores<QT>(tile + lo.k, qf, s);
            tile_softmax<QT>(s, p, lsum);
            tile_pv<QT>(tile + lo.v[0], tile + lo.v[1], p, oacc);
            count_masked(it);
            cur = cur + 1 == STAGES ? 0 : cur + 1;
        }
    }
    sync_tile<0>();  // no DMA in flight, every wave done with the ring

    if constexpr (KS == 1) {
        // One key stream: each wave owns its queries' sums outright. Lane
        // holds O^T[d = 32*dt + 8*rb + 4*h + 0..3][query 32*qt + (lane & 31)].
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            const int row = qbase + 32 * qt + (lane & 31);
            const float l = lsum[qt] + __shfl_xor(lsum[qt], 32) - masked;
            if (row >= M) continue;
            if (nsplit == 1) {
                _Float16 *dst = o + ((size_t)b * M + row) * HD + 4 * h;
#pragma unroll
                for (int dt = 0; dt < 2; ++dt)
#pragma unroll
                    for (int rb = 0; rb < 4; ++rb) {
                        half4 hv;
#pragma unroll
                        for (int y = 0; y < 4; ++y) hv[y] = (_Float16)(oacc[dt][qt][4 * rb + y] / l);
                        *(half4 *)(dst + 32 * dt + 8 * rb) = hv;
                    }
            } else {
                const size_t prow = ((size_t)split * B + b) * M + row;
                float *dst = ws_w + prow * HD + 4 * h;
#pragma unroll
                for (int dt = 0; dt < 2; ++dt)
#pragma unroll
                    for (int rb = 0; rb < 4; ++rb)
                        *(float4v *)(dst + 32 * dt + 8 * rb) =
                            float4v{oacc[dt][qt][4 * rb], oacc[dt][qt][4 * rb + 1], oacc[dt][qt][4 * rb + 2],
                                    oacc[dt][qt][4 * rb + 3]};
                if (h == 0) ws_l[prow] = l;
            }
        }
    } else {
        // Sum the KS streams of each query group in LDS (fixed order), then
        // write O (one split) or the partial W, L.
        {
            char *reg = smem + wave * C::RED_BYTES;
            float *lreg = (float *)(reg + 32 * QT * RED_ROW_BYTES);
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                const int qr = 32 * qt + (lane & 31);
#pragma unroll
                for (int dt = 0; dt < 2; ++dt)
#pragma unroll
                    for (int rb = 0; rb < 4; ++rb) {
                        const int d = 32 * dt + 8 * rb + 4 * h;
                        *(float4v *)(reg + qr * RED_ROW_BYTES + d * 4) =
                            float4v{oacc[dt][qt][4 * rb], oacc[dt][qt][4 * rb + 1], oacc[dt][qt][4 * rb + 2],
                                    oacc[dt][qt][4 * rb + 3]};
                    }
                const float lfull = lsum[qt] + __shfl_xor(lsum[qt], 32) - masked;
                if (h == 0) lreg[qr] = lfull;
            }
        }
        __syncthreads();
        if (qbase >= M) return;
        const int qr = lane % (32 * QT);
        const int d0 = ks * C::DW + (lane / (32 * QT)) * C::VPL;
        float acc[C::VPL];
#pragma unroll
        for (int x = 0; x < C::VPL; ++x) acc[x] = 0.f;
        float l = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            const char *reg = smem + (qw * KS + s2) * C::RED_BYTES;
            const float *lreg = (const float *)(reg + 32 * QT * RED_ROW_BYTES);
#pragma unroll
            for (int x = 0; x < C::VPL; x += 4) {
                const float4v t = *(const float4v *)(reg + qr * RED_ROW_BYTES + (d0 + x) * 4);
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
                const size_t prow = ((size_t)split * B + b) * M + row;
                float *dst = ws_w + prow * HD + d0;
#pragma unroll
                for (int x = 0; x < C::VPL; x += 4)
                    *(float4v *)(dst + x) = float4v{acc[x], acc[x + 1], acc[x + 2], acc[x + 3]};
                if (ks == 0 && d0 == 0) ws_l[prow] = l;
            }
        }
    }
}

// Combine: 16 threads per output row, 4 head dims each; sums in split order.
__global__ __launch_bounds__(256) void gqa_combine_kernel(const float *__restrict__ ws_w,
                                                          const float *__restrict__ ws_l,
                                                          _Float16 *__restrict__ o, long long rows,
                                                          int nsplit) {
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long row = gid >> 4;
    const int c = (int)(gid & 15);
    if (row >= rows) return;
    float l = 0.f;
    float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int s = 0; s < nsplit; ++s) {
        const long long prow = (long long)s * rows + row;
        l += ws_l[prow];
        acc += *reinterpret_cast<const float4v *>(ws_w + prow * HD + 4 * c);
    }
    half4 hv;
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = (_Float16)(acc[i] / l);
    *reinterpret_cast<half4 *>(o + row * HD + 4 * c) = hv;
}

template <int QT, int QW, int KS>
int launch_partial_cfg(const mga::Plan &p, const _Float16 *q, const _Float16 *k, const _Float16 *v,
                       _Float16 *o, float *w, float *l, hipStream_t st) {
    const int pairs = p.B * p.splits;
    const int groups = (pairs + 7) / 8;
    const dim3 grid((unsigned)(groups * 8 * p.mtiles));
    hipLaunchKernelGGL((gqa_partial_kernel<QT, QW, KS>), grid, dim3(64 * QW * KS), 0, st, q, k, v, o,
                       w, l, p.B, p.M, p.N, p.chunk_keys, p.splits, p.mtiles);
    return (int)hipGetLastError();
}

}  // namespace

namespace mga {

static void ws_split(const Plan &p, const void *ws, float **w, float **l) {
    *w = (float *)ws;
    *l = (float *)((char *)ws + (size_t)p.splits * p.B * p.M * HD * sizeof(float));
}

int launch_partial(const Plan &p, const void *q, const void *k, const void *v, void *o,
                   void *ws, void *stream) {
    float *w = nullptr, *l = nullptr;
    if (p.splits > 1) ws_split(p, ws, &w, &l);
    hipStream_t st = (hipStream_t)stream;
    const _Float16 *qh = (const _Float16 *)q, *kh = (const _Float16 *)k, *vh = (const _Float16 *)v;
    _Float16 *oh = (_Float16 *)o;
    switch (p.variant) {
    case kVariantDecode: return launch_partial_cfg<1, 1, 8>(p, qh, kh, vh, oh, w, l, st);
    case kVariantSmall: return launch_partial_cfg<2, 1, 8>(p, qh, kh, vh, oh, w, l, st);
    case kVariantMedium: return launch_partial_cfg<2, 2, 4>(p, qh, kh, vh, oh, w, l, st);
    default: return launch_partial_cfg<2, 4, 2>(p, qh, kh, vh, oh, w, l, st);
    }
}

int launch_combine(const Plan &p, void *o, const void *ws, void *stream) {
    float *w = nullptr, *l = nullptr;
    ws_split(p, ws, &w, &l);
    const long long rows = (long long)p.B * p.M;
    const long long threads = rows * 16;
    const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(gqa_combine_kernel, grid, dim3(kThreads), 0, (hipStream_t)stream, w, l,
                       (_Float16 *)o, rows, p.splits);
    return (int)hipGetLastError();
}

}  // namespace mga
