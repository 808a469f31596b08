// Split-KV partial kernel and combine kernel for the GQA exp-sum-div graph on
// gfx950 (MI355X, CDNA4).
//
// Graph (Mirage GQA tutorial, "Mirage: Define GQA Computation Graph"):
//   A = Q K, E = exp(A), S = rowsum(E), O = (E / S) V   -- no scale, no max.
// Split-KV form (kaispace blog, sections 2.1 and 4.2-4.3: a for-loop over the
// key dimension that accumulates, followed by a combine block graph): each
// workgroup owns one (batch row b, query tile, key chunk) and accumulates
//   W = sum_n fp16(e_n) V[n]   and   L = sum_n fp16(e_n)
// over its chunk; O = sum_s W_s / sum_s L_s. With no running maximum the
// partials combine by plain sums.
//
// Partial kernel, per workgroup of 4 waves (256 threads):
//   * pre-loop: each wave keeps Q for its 16*QG query rows in registers as
//     MFMA B operands (Q^T fragments, 8 consecutive head-dim values a lane).
//   * loop over 128-key blocks of its chunk, double-buffered in LDS: global
//     16-byte loads of the next block are in flight while the current block
//     is computed. K (head-dim-major in HBM) is stored to LDS as K^T rows
//     [key][64 d]; V (key-major in HBM) is stored as V^T rows [d][128 keys].
//     Both need a 16-bit transpose, done in registers (8x8 tiles) between the
//     global load and the LDS store.
//   * S^T = K^T Q^T on v_mfma_f32_16x16x32_f16 (keys on the accumulator's
//     row axis, queries on its column axis), E = exp2(S * log2 e) in fp32,
//     P = fp16(E) (round toward zero, packed), then O^T += V^T P^T on the same
//     MFMA. In the 16x16 accumulator layout a lane holds 4 consecutive keys
//     of one query, so two key tiles give exactly the 8 k-slots a lane feeds
//     to the next MFMA's B operand: the scores never leave registers. The
//     V^T LDS layout orders keys inside each 32-key group to match those
//     k-slots. The row-sum L comes from one more MFMA whose A operand is all
//     ones, so it sums the very fp16 P the numerator used.
//   * post-loop: with one split, O = fp16(W / L) is stored directly; otherwise
//     W (fp32, 64 per row) and L (fp32) go to the caller's workspace.
// Tails: keys past the chunk end are never loaded (zero-filled) and their E
// is forced to 0 (a zero-filled K column would give exp(0) = 1); query rows
// past M are zero-filled and never stored.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mga_internal.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int KB = mga::kKeyBlock;            // keys per stage
constexpr int HD = mga::kHeadDim;             // head dim
constexpr int STAGE_HALVES = 2 * KB * HD;     // K^T + V^T per stage
constexpr float LOG2E = 1.4426950408889634f;

// K^T tile: [128 keys][64 d], 128-byte rows of eight 16-byte chunks. The
// chunk index is XOR-swizzled by the row so that the 16 lanes reading one
// chunk column of 16 consecutive rows hit distinct banks for either 32 or
// 64 banks of 4 bytes.
__device__ __forceinline__ int kt_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int kt_off(int row, int chunk) {
    return row * HD + ((chunk ^ kt_swz(row)) << 3);
}
// V^T tile: [64 d][128 key slots], 256-byte rows of sixteen 16-byte chunks,
// chunk index XOR-swizzled by (row & 15).
__device__ __forceinline__ int vt_off(int row, int chunk) {
    return row * KB + ((chunk ^ (row & 15)) << 3);
}

// Pack half `sel` (0 = low, 1 = high) of a and b into one dword (a's half low).
__device__ __forceinline__ uint32_t pick_pair(uint32_t a, uint32_t b, int sel) {
    return sel ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

// 8x8 transpose of 16-bit elements held as 8 rows of 16 bytes:
// out[c] = { in[0][c], in[1][c], ..., in[7][c] }.
__device__ __forceinline__ void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
            out[c][p] = pick_pair(in[2 * p][c >> 1], in[2 * p + 1][c >> 1], c & 1);
    }
}

// Global -> registers for one 128-key block starting at key kb0.
// Threads 0..127 take K: thread (dgrp = t & 7, ngrp = t >> 3) loads the 8 K
// rows d = 8*dgrp .. +7 at keys kb0 + 8*ngrp .. +7.
// Threads 128..255 take V: thread (kset = t & 15, dgrp = t >> 4) loads the 8 V
// rows of key set kset (keys 32*(kset>>2) + 16*(j>>2) + 4*(kset&3) + (j&3),
// j = 0..7) at head dims 8*dgrp .. +7.
__device__ __forceinline__ void stage_load(u32x4 r[8], const _Float16 *__restrict__ kb_ptr,
                                           const _Float16 *__restrict__ vb_ptr, int N, int kb0,
                                           int kend, int tid) {
    if (tid < 128) {
        const int dgrp = tid & 7, ngrp = tid >> 3;
        const int key0 = kb0 + 8 * ngrp;
        const bool ok = key0 < kend;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const _Float16 *src = kb_ptr + (size_t)(8 * dgrp + i) * N + key0;
            r[i] = ok ? *reinterpret_cast<const u32x4 *>(src) : u32x4{0u, 0u, 0u, 0u};
        }
    } else {
        const int t = tid - 128;
        const int kset = t & 15, dgrp = t >> 4;
        const int kbase = kb0 + 32 * (kset >> 2) + 4 * (kset & 3);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = kbase + 16 * (j >> 2) + (j & 3);
            const _Float16 *src = vb_ptr + (size_t)key * HD + 8 * dgrp;
            r[j] = key < kend ? *reinterpret_cast<const u32x4 *>(src) : u32x4{0u, 0u, 0u, 0u};
        }
    }
}

// Registers -> LDS (transposed) for the block loaded by stage_load.
__device__ __forceinline__ void stage_store(const u32x4 r[8], _Float16 *__restrict__ stage,
                                            int tid) {
    u32x4 t8[8];
    transpose8x8(r, t8);
    if (tid < 128) {
        const int dgrp = tid & 7, ngrp = tid >> 3;
        _Float16 *kt = stage;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int row = 8 * ngrp + j;  // local key
            *reinterpret_cast<u32x4 *>(kt + kt_off(row, dgrp)) = t8[j];
        }
    } else {
        const int t = tid - 128;
        const int kset = t & 15, dgrp = t >> 4;
        _Float16 *vt = stage + KB * HD;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int row = 8 * dgrp + c;  // head dim
            *reinterpret_cast<u32x4 *>(vt + vt_off(row, kset)) = t8[c];
        }
    }
}

// One 128-key block for one wave: 16*QG queries x 128 keys.
template <int QG, bool MASK>
__device__ __forceinline__ void compute_block(const _Float16 *__restrict__ stage,
                                              const half8 (&qf)[QG][2], float4v (&oacc)[4][QG],
                                              float4v (&lacc)[QG], int r16, int g, int kb0,
                                              int kend) {
    const _Float16 *kt = stage;
    const _Float16 *vt = stage + KB * HD;
    const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
    for (int kb = 0; kb < KB / 32; ++kb) {
        float4v s[2][QG];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int row = 16 * (2 * kb + tt) + r16;
            const half8 a0 = *reinterpret_cast<const half8 *>(kt + kt_off(row, g));
            const half8 a1 = *reinterpret_cast<const half8 *>(kt + kt_off(row, 4 + g));
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
                float4v c = {0.f, 0.f, 0.f, 0.f};
                c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qf[qg][0], c, 0, 0, 0);
                s[tt][qg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qf[qg][1], c, 0, 0, 0);
            }
        }
        half8 p[QG];
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
            float e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float x = __builtin_amdgcn_exp2f(s[j >> 2][qg][j & 3] * LOG2E);
                if (MASK) {
                    const int key = kb0 + 32 * kb + 16 * (j >> 2) + 4 * g + (j & 3);
                    x = key < kend ? x : 0.f;
                }
                e[j] = x;
            }
            u32x4 packed;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                packed[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(e[2 * j], e[2 * j + 1]));
            p[qg] = __builtin_bit_cast(half8, packed);
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const half8 av = *reinterpret_cast<const half8 *>(vt + vt_off(16 * dt + r16, 4 * kb + g));
#pragma unroll
            for (int qg = 0; qg < QG; ++qg)
                oacc[dt][qg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, p[qg], oacc[dt][qg], 0, 0, 0);
        }
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
            lacc[qg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, p[qg], lacc[qg], 0, 0, 0);
    }
}

template <int QG>
__global__ __launch_bounds__(256) void gqa_partial_kernel(
    const _Float16 *__restrict__ q, const _Float16 *__restrict__ k,
    const _Float16 *__restrict__ v, _Float16 *__restrict__ o, float *__restrict__ ws_w,
    float *__restrict__ ws_l, int B, int M, int N, int chunk_keys, int nsplit) {
    __shared__ __attribute__((aligned(16))) _Float16 smem[2 * STAGE_HALVES];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int r16 = lane & 15, g = lane >> 4;
    const int split = blockIdx.x, mtile = blockIdx.y, b = blockIdx.z;

    const int kstart = split * chunk_keys;
    const int kend = min(N, kstart + chunk_keys);
    const int nblk = (kend - kstart + KB - 1) / KB;

    const _Float16 *kb_ptr = k + (size_t)b * HD * N;
    const _Float16 *vb_ptr = v + (size_t)b * N * HD;

    const int qrow0 = mtile * 64 * QG + wave * 16 * QG;
    const bool active = qrow0 < M;

    // Pre-loop: Q^T fragments (B operand): lane holds query qrow0+16*qg+r16,
    // head dims 32*ks + 8*g .. +7.
    half8 qf[QG][2];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        const int row = qrow0 + 16 * qg + r16;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            if (row < M)
                qf[qg][ks] = *reinterpret_cast<const half8 *>(q + ((size_t)b * M + row) * HD + 32 * ks + 8 * g);
            else
                qf[qg][ks] = half8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }

    float4v oacc[4][QG];
    float4v lacc[QG];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        lacc[qg] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[dt][qg] = float4v{0.f, 0.f, 0.f, 0.f};
    }

    u32x4 r[8];
    stage_load(r, kb_ptr, vb_ptr, N, kstart, kend, tid);
    stage_store(r, smem, tid);
    __syncthreads();

    for (int it = 0; it < nblk; ++it) {
        const int kb0 = kstart + it * KB;
        const bool more = it + 1 < nblk;
        if (more) stage_load(r, kb_ptr, vb_ptr, N, kb0 + KB, kend, tid);
        const _Float16 *cur = smem + (it & 1) * STAGE_HALVES;
        if (active) {
            if (kb0 + KB <= kend)
                compute_block<QG, false>(cur, qf, oacc, lacc, r16, g, kb0, kend);
            else
                compute_block<QG, true>(cur, qf, oacc, lacc, r16, g, kb0, kend);
        }
        if (more) stage_store(r, smem + ((it + 1) & 1) * STAGE_HALVES, tid);
        __syncthreads();
    }

    if (!active) return;

    // Post-loop. Accumulator layout: lane holds O^T[d = 16*dt + 4*g + i][query r16];
    // every element of lacc[qg] holds L for query r16.
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        const int row = qrow0 + 16 * qg + r16;
        if (row >= M) continue;
        if (nsplit == 1) {
            const float l = lacc[qg][0];
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                half4 h;
#pragma unroll
                for (int i = 0; i < 4; ++i) h[i] = (_Float16)(oacc[dt][qg][i] / l);
                *reinterpret_cast<half4 *>(o + ((size_t)b * M + row) * HD + 16 * dt + 4 * g) = h;
            }
        } else {
            const size_t prow = ((size_t)split * B + b) * M + row;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                *reinterpret_cast<float4v *>(ws_w + prow * HD + 16 * dt + 4 * g) = oacc[dt][qg];
            if (g == 0) ws_l[prow] = lacc[qg][0];
        }
    }
}

// Combine: 16 threads per output row, 4 head dims each; sums in split order.
__global__ __launch_bounds__(256) void gqa_combine_kernel(const float *__restrict__ ws_w,
                                                          const float *__restrict__ ws_l,
                                                          _Float16 *__restrict__ o, long long rows,
                                                          int nsplit) {
    const size_t gid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t row = gid >> 4;
    const int c = (int)(gid & 15);
    if (row >= (size_t)rows) return;
    float l = 0.f;
    float4v acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nsplit; ++s) {
        const size_t prow = (size_t)s * rows + row;
        l += ws_l[prow];
        acc += *reinterpret_cast<const float4v *>(ws_w + prow * HD + 4 * c);
    }
    half4 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = (_Float16)(acc[i] / l);
    *reinterpret_cast<half4 *>(o + row * HD + 4 * c) = h;
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
    const dim3 grid(p.splits, p.mtiles, p.B);
    const dim3 block(kThreads);
    hipStream_t st = (hipStream_t)stream;
    const _Float16 *qh = (const _Float16 *)q, *kh = (const _Float16 *)k, *vh = (const _Float16 *)v;
    _Float16 *oh = (_Float16 *)o;
    switch (p.qgroups) {
    case 1:
        hipLaunchKernelGGL(gqa_partial_kernel<1>, grid, block, 0, st, qh, kh, vh, oh, w, l, p.B,
                           p.M, p.N, p.chunk_keys, p.splits);
        break;
    case 2:
        hipLaunchKernelGGL(gqa_partial_kernel<2>, grid, block, 0, st, qh, kh, vh, oh, w, l, p.B,
                           p.M, p.N, p.chunk_keys, p.splits);
        break;
    default:
        hipLaunchKernelGGL(gqa_partial_kernel<4>, grid, block, 0, st, qh, kh, vh, oh, w, l, p.B,
                           p.M, p.N, p.chunk_keys, p.splits);
        break;
    }
    return (int)hipGetLastError();
}

int launch_combine(const Plan &p, void *o, const void *ws, void *stream) {
    float *w = nullptr, *l = nullptr;
    ws_split(p, ws, &w, &l);
    const size_t rows = (size_t)p.B * p.M;
    const size_t threads = rows * 16;
    const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
    hipLaunchKernelGGL(gqa_combine_kernel, grid, dim3(kThreads), 0, (hipStream_t)stream, w, l,
                       (_Float16 *)o, (long long)rows, p.splits);
    return (int)hipGetLastError();
}

}  // namespace mga
