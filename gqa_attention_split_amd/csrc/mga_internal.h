// Internal declarations shared by the host dispatch and the kernel launchers.
#pragma once

#include <stddef.h>

namespace mga {

// Element strides of one call. Q[b][i][d] at q + b*q_b + i*q_i + d,
// V[b][n][d] at v + b*v_b + n*v_n + d, O[b][i][d] at o + b*o_b + i*o_i + d;
// K[b][d][n] at k + b*k_b + d*k_r + n (head-dim-major) or k + b*k_b + n*k_r + d
// (key-major). Row strides are below 2^30 (checked with the byte extents).
struct Strides {
    long long q_b, k_b, v_b, o_b;
    int q_i, k_r, v_n, o_i;
};

// Geometry of one launch, decided on the host before anything is enqueued.
struct Plan {
    int B, M, N, D;
    bool key_major;   // K stored [N][D] per batch (else [D][N])
    bool qknorm;      // rms_norm of Q rows and key vectors before the graph
    float eps;        // rms_norm epsilon (qknorm only)
    bool repack;      // contiguous K with N % 8 != 0: copied first to rows of ceil8(N) keys
    size_t repack_off;  // byte offset of that copy in the workspace
    Strides st;
    int variant;      // kernel shape, one of the kVariant* values
    int tile_rows;    // query rows per workgroup
    int mtiles;       // ceil(M / tile_rows)
    int nblocks;      // ceil(N / key block)
    int splits;       // effective split count (>= 1)
    int chunk_keys;   // keys per split (a multiple of the key block)
    size_t ws_bytes;  // workspace the plan needs (0 when splits == 1)
};

// Kernel shapes: (query tiles of 32 per wave, query waves, key streams).
// Shapes have 8 waves per workgroup (two per SIMD) except the 32-row one
// (4 waves; two such workgroups share a CU) and head dim 128 (2 waves).
constexpr int kVariantDecode = 0;  // (1, 1, 4),  32 rows per workgroup, 4 waves, wave-private rings
constexpr int kVariantSmall = 1;   // (2, 1, 8),  64 rows per workgroup, wave-private rings
constexpr int kVariantMedium = 2;  // (2, 2, 4), 128 rows per workgroup, shared ring
constexpr int kVariantLarge = 3;   // (2, 4, 2), 256 rows per workgroup, shared ring
// Head dim 128: (1, 1, 2), 32 rows per workgroup, 2 waves with wave-private
// rings of two 16 KiB tiles.
constexpr int kVariantDecode128 = 4;
// (1, 2, 4): 64 rows per workgroup on a shared ring, for split key ranges:
// its cross-stream reduction sums 4 streams of 32-row partials, not 8 of
// 64-row ones.
constexpr int kVariantSmallShared = 5;

constexpr int kKeyBlock = 128;
// Buffer descriptors address one batch's K or V with 32-bit byte offsets:
// D * N * 2 bytes stay below 2^31.
constexpr int max_keys(int D) { return (1 << 30) / D - 1; }
constexpr int kThreads = 256;
// Split count from which the combine runs four split groups per
// workgroup (gqa_combine_grouped_kernel, which needs kThreads == 256). Cold
// A/B, us per forward: (2, 256, 32768) at 32 splits 16.10 -> 14.53; at 8
// splits (2, 256, 4096) 7.54 -> 7.77 and (64, 8, 8192) 27.89 -> 28.26, at 16
// splits (16, 1, 16384, 128) 29.20 -> 29.46, so fewer splits keep the
// one-group form.
constexpr int kGroupedCombineSplits = 32;
static_assert(kThreads == 256, "grouped combine: four groups of 64 threads");

// Fills `p` for a call; returns an mga_status (0 = ok). Host only; its one
// runtime query is device_cus() (the chip size the split policy fills).
// The layout is left contiguous and unchecked; set_layout fixes it. With
// qknorm the kernel shape comes from the wave-private-ring shapes only.
int make_plan(int B, int M, int N, int D, int splits, Plan *p, bool qknorm = false);

// Checks the nine element strides (q_b, q_i, k_b, k_d, k_n, v_b, v_n, o_b,
// o_i; NULL = contiguous) against the plan's shape and stores them. Returns
// an mga_status. NULL with N % 8 != 0 plans the K repack (and grows
// ws_bytes by its size).
int set_layout(Plan *p, const long long *strides);

// Argument checks shared by every entry point (host only).
int check_call(const void *q, const void *k, const void *v, const void *o, const Plan &p,
               const void *ws, size_t ws_bytes, bool need_inputs);

// Bytes of the fixed device scratch behind mga_gqa_forward_noalloc.
constexpr size_t kScratchBytes = (size_t)16 << 20;
// Address of that scratch on the current device (looked up once per device);
// 0 or a hipError_t value.
int scratch_ptr(void **out);

// Compute units of the current device (mga_device.cpp; looked up once per
// device); the split policy sizes the grid to them. kDefaultCUs (MI355X in
// its default single-partition mode) when no device answers, e.g. on a host
// without a GPU.
constexpr int kDefaultCUs = 256;
int device_cus();

// Kernel launchers (gqa_kernels.hip). Return 0 or a hipError_t value.
int launch_partial(const Plan &p, const void *q, const void *k, const void *v, void *o,
                   void *ws, void *stream);
int launch_combine(const Plan &p, void *o, const void *ws, void *stream);
// Copies K [B][D][N] into the workspace as [B][D][ceil8(N)] (padding zero).
int launch_repack(const Plan &p, const void *k, void *ws, void *stream);

}  // namespace mga
