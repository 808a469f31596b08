// Host side of the C ABI: argument checks, split policy, workspace sizing and
// the two launches. See include/mga_gqa.h for the contract of each entry point.
//
// The split count is a grid-dimension choice (the kaispace blog, section 4.2,
// describes the grid and for-loop ranges as search parameters; here a fixed
// rule picks them), and the workspace plays the role of the runtime buffer
// whose size the CUDA transpiler reports (blog section 5.2) and that the
// generated entry point receives as its `buf` argument (Mirage docs,
// "Generated CUDA Code Example").

#include <stdint.h>

#include <algorithm>
#include <climits>
#include <cmath>

#include "../../include/mga_gqa.h"
#include "mga_internal.h"

namespace mga {

namespace {

inline long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

constexpr long long kMinChunkBlocks = 4;
// Most splits the policy uses for N keys.
long long max_splits(int N) { return std::max(1LL, ceil_div(N, kKeyBlock) / kMinChunkBlocks); }

int rows_for(int variant) {
    switch (variant) {
    case kVariantDecode:
    case kVariantDecode128: return 32;
    case kVariantSmall:
    case kVariantSmallShared: return 64;
    case kVariantMedium: return 128;
    default: return 256;
    }
}

// Query rows per workgroup, for a chip of `cus` compute units (one 8-wave
// workgroup fills one). The rule comes from cold-input tile x split sweeps of
// the five benchmark shapes on MI355X (256 compute units):
//   * a tile shape that fills the chip (a workgroup per CU) without splitting
//     beats any split configuration: 256 rows, else 128 rows;
//   * else 256-row tiles if two splits fill the chip;
//   * else 64-row tiles with key splits, unless even the most splits the key
//     count allows leave them short of the chip: then 32-row tiles, which
//     double the workgroups. (At an equal, full workgroup count, 64-row tiles
//     with twice the splits beat 32-row tiles: half the K/V bytes per
//     workgroup.)
// Rows M <= 32 take 32-row tiles. The QK-normalised path has only the 32-
// and 64-row shapes (the 64-row one on the shared ring once keys are split).
int variant_for(int B, int M, int N, int D, bool qknorm, long long cus) {
    if (D == 128) return kVariantDecode128;
    if (qknorm) return M <= 32 ? kVariantDecode : kVariantSmall;  // 32 or 64 rows
    if (M <= 32) return kVariantDecode;
    const long long b = B, ms = max_splits(N);
    if (M > 128 && b * ceil_div(M, 256) >= cus) return kVariantLarge;
    if (M > 64 && b * ceil_div(M, 128) >= cus) return kVariantMedium;
    if (M > 128 && b * ceil_div(M, 256) * std::min(2LL, ms) >= cus) return kVariantLarge;
    if (b * ceil_div(M, 64) * ms >= cus) return kVariantSmall;
    return kVariantDecode;
}

// Workgroups of a shape that fit one compute unit at once: the 32-row shape
// has 4 waves and 64-70 KB of LDS (with or without QK norm), so two fit;
// every other shape takes a whole CU at the policy's split counts.
long long wgs_per_cu(int variant) { return variant == kVariantDecode ? 2 : 1; }

// Policy: split the keys just enough that the grid fills every compute unit
// (one or two workgroups each), keeping at least kMinChunkBlocks key blocks
// per split where N allows (shorter chunks cost more in partial traffic and
// combine work than the extra workgroups gain).
int policy_splits(int B, int M, int N, int variant, long long cus) {
    if (N < 1 || B < 1 || M < 1) return 1;
    const long long base = (long long)B * ceil_div(M, rows_for(variant));
    const long long s = std::min(ceil_div(cus * wgs_per_cu(variant), base), max_splits(N));
    return (int)std::max(1LL, s);
}

bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

}  // namespace

int make_plan(int B, int M, int N, int D, int splits, Plan *p, bool qknorm) {
    if (B < 0 || M < 0 || N < 1 || splits < 0) return MGA_ERR_INVALID_VALUE;
    if (D != 64 && D != 128) return MGA_ERR_CONFIG;
    const long long nblocks = ceil_div(N, kKeyBlock);
    if (splits > nblocks) return MGA_ERR_CONFIG;
    p->B = B;
    p->M = M;
    p->N = N;
    p->D = D;
    const long long cus = device_cus();
    p->variant = variant_for(B, M, N, D, qknorm, cus);
    p->qknorm = qknorm;
    p->eps = 0.f;
    p->repack = false;
    p->repack_off = 0;
    p->tile_rows = rows_for(p->variant);
    p->mtiles = (int)ceil_div(M, p->tile_rows);
    p->nblocks = (int)nblocks;
    p->key_major = false;
    p->st = Strides{(long long)M * D, (long long)D * N, (long long)N * D, (long long)M * D, D, N, D, D};
    const int want = splits == 0 ? policy_splits(B, M, N, p->variant, cus) : splits;
    const long long chunk_blocks = ceil_div(nblocks, want);
    p->splits = (int)ceil_div(nblocks, chunk_blocks);
    p->chunk_keys = (int)(chunk_blocks * kKeyBlock);
    // 64-row tiles over split key ranges run on the shared ring (the plain
    // and the QK-normalised path alike). With a short key
    // stream per workgroup its smaller end-of-kernel reduction wins (cold
    // A/B: 7% at (16, 256, 4096) x 4 splits and (2, 256, 32768) x 32); an
    // unsplit stream keeps the private ring (2% faster at (64, 256, 4096)).
    if (p->variant == kVariantSmall && p->splits > 1) p->variant = kVariantSmallShared;
    if (N > max_keys(D)) return MGA_ERR_CONFIG;
    const long long groups = ceil_div((long long)B * p->splits, 8) * 8 * p->mtiles;
    if (groups > INT_MAX || (long long)B * M > INT_MAX / D) return MGA_ERR_CONFIG;
    if (p->splits > 1) {
        // o_s fp16 [splits][B][M][D] rounded up to 256 bytes, then L_s fp32 [splits][B][M]
        const size_t rows = (size_t)p->splits * B * M;
        const size_t o_bytes = (rows * D * 2 + 255) & ~(size_t)255;
        p->ws_bytes = (o_bytes + rows * sizeof(float) + 255) & ~(size_t)255;
    } else {
        p->ws_bytes = 0;
    }
    return MGA_OK;
}

int set_layout(Plan *p, const long long *s) {
    const long long B = p->B, M = p->M, N = p->N, D = p->D;
    long long q_b, q_i, k_b, k_d, k_n, v_b, v_n, o_b, o_i;
    if (s) {
        q_b = s[0], q_i = s[1], k_b = s[2], k_d = s[3], k_n = s[4];
        v_b = s[5], v_n = s[6], o_b = s[7], o_i = s[8];
    } else {
        q_b = M * D, q_i = D, k_b = D * N, k_d = N, k_n = 1, v_b = N * D, v_n = D, o_b = M * D, o_i = D;
        if (N % 8 != 0) {
            // Contiguous K rows start 2-byte aligned only: the partial kernel
            // reads a copy with rows of ceil8(N) keys from the workspace.
            const long long n8 = (N + 7) & ~7LL;
            p->repack = true;
            p->repack_off = p->ws_bytes;
            p->ws_bytes += ((size_t)(B * D * n8) * 2 + 255) & ~(size_t)255;
            k_b = D * n8, k_d = n8;
        }
    }
    // Row strides up to 2^30 and batch strides up to 2^48 elements keep every
    // product below 2^63; the byte extents are checked against 2^31 below.
    const long long row_max = 1LL << 30, batch_max = 1LL << 48;
    for (long long x : {q_b, q_i, k_b, k_d, k_n, v_b, v_n, o_b, o_i})
        if (x < 0) return MGA_ERR_LAYOUT;
    for (long long r : {q_i, k_d, k_n, v_n, o_i})
        if (r > row_max) return MGA_ERR_CONFIG;
    for (long long b : {q_b, k_b, v_b, o_b})
        if (b > batch_max) return MGA_ERR_CONFIG;
    // Every 16-byte DMA unit and output store stays aligned: strides other
    // than the unit one are multiples of 8 elements.
    auto al = [](long long x) { return x % 8 == 0; };
    bool km;
    if (k_n == 1 && k_d >= N && al(k_d))
        km = false;  // K[d][n]: head-dim-major rows of at least N keys
    else if (k_d == 1 && k_n >= D && al(k_n))
        km = true;   // K[n][d]: key-major rows of at least D head dims
    else
        return MGA_ERR_LAYOUT;
    if (!al(q_b) || !al(k_b) || !al(v_b) || !al(o_b)) return MGA_ERR_LAYOUT;
    if (!al(q_i) || !al(v_n) || !al(o_i) || q_i < D || v_n < D || o_i < D) return MGA_ERR_LAYOUT;
    if (B > 1 && M > 0 && o_b < (M - 1) * o_i + D) return MGA_ERR_LAYOUT;  // O batches overlap
    // Byte extents behind one buffer descriptor: a batch's K and V from the
    // first key on, and a workgroup's Q rows. A head-dim-major K descriptor
    // ends at the 16-byte unit that holds key N - 1 of the last row.
    const long long lim = 1LL << 31;
    const long long k_ext = km ? (N - 1) * k_n + D : (D - 1) * k_d + ((N + 7) & ~7LL);
    if (2 * k_ext >= lim || 2 * ((N - 1) * v_n + D) >= lim) return MGA_ERR_CONFIG;
    if (2 * ((p->tile_rows - 1) * q_i + D) >= lim) return MGA_ERR_CONFIG;
    p->key_major = km;
    p->st = Strides{q_b, k_b, v_b, o_b, (int)q_i, (int)(km ? k_n : k_d), (int)v_n, (int)o_i};
    return MGA_OK;
}

int check_call(const void *q, const void *k, const void *v, const void *o, const Plan &p,
               const void *ws, size_t ws_bytes, bool need_inputs) {
    if (p.B == 0 || p.M == 0) return MGA_OK;
    if (!o || (need_inputs && (!q || !k || !v))) return MGA_ERR_INVALID_VALUE;
    if (misaligned(o) || (need_inputs && (misaligned(q) || misaligned(k) || misaligned(v))))
        return MGA_ERR_LAYOUT;
    if (p.ws_bytes > 0 && (!ws || misaligned(ws) || ws_bytes < p.ws_bytes))
        return MGA_ERR_WORKSPACE;
    return MGA_OK;
}

}  // namespace mga

extern "C" {

const char *mga_status_string(int status) {
    switch (status) {
    case MGA_OK: return "MGA_OK: success";
    case MGA_ERR_INVALID_VALUE:
        return "MGA_ERR_INVALID_VALUE: null pointer, negative B/M/splits, or N < 1";
    case MGA_ERR_LAYOUT:
        return "MGA_ERR_LAYOUT: pointer not 16-byte aligned, or a stride not allowed";
    case MGA_ERR_CONFIG:
        return "MGA_ERR_CONFIG: head dim not 64 or 128, splits above ceil(N/128), N above 2^30/D - 1, "
               "a stride or byte extent too large, or a grid too large";
    case MGA_ERR_WORKSPACE: return "MGA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MGA_ERR_HIP: return "MGA_ERR_HIP: kernel launch failed";
    case MGA_ERR_SCRATCH:
        return "MGA_ERR_SCRATCH: the call needs more workspace than the 16 MiB device scratch of "
               "mga_gqa_forward_noalloc holds";
    default: return "unknown mga status";
    }
}

int mga_gqa_choose_splits(int B, int M, int N, int D) {
    mga::Plan p;
    if (mga::make_plan(B, M, N, D, 0, &p) != MGA_OK) return 1;
    return p.splits;
}

int mga_gqa_effective_splits(int B, int M, int N, int D, int splits) {
    mga::Plan p;
    if (mga::make_plan(B, M, N, D, splits, &p) != MGA_OK) return -1;
    return p.splits;
}

size_t mga_gqa_workspace_bytes(int B, int M, int N, int D, int splits) {
    mga::Plan p;
    if (mga::make_plan(B, M, N, D, splits, &p) != MGA_OK) return 0;
    if (mga::set_layout(&p, nullptr) != MGA_OK) return 0;
    return p.ws_bytes;
}

int mga_gqa_check_args(const void *q, const void *k, const void *v, const void *o, int B, int M,
                       int N, int D, int splits, const void *ws, size_t ws_bytes) {
    return mga_gqa_check_args_strided(q, k, v, o, B, M, N, D, nullptr, splits, ws, ws_bytes);
}

int mga_gqa_check_args_strided(const void *q, const void *k, const void *v, const void *o, int B,
                               int M, int N, int D, const int64_t *strides, int splits,
                               const void *ws, size_t ws_bytes) {
    static_assert(sizeof(long long) == sizeof(int64_t), "stride width");
    mga::Plan p;
    int rc = mga::make_plan(B, M, N, D, splits, &p);
    if (rc == MGA_OK) rc = mga::set_layout(&p, reinterpret_cast<const long long *>(strides));
    if (rc != MGA_OK) return rc;
    return mga::check_call(q, k, v, o, p, ws, ws_bytes, true);
}

int mga_gqa_partial(const void *q, const void *k, const void *v, void *o, int B, int M, int N,
                    int D, int splits, void *ws, size_t ws_bytes, void *stream) {
    mga::Plan p;
    int rc = mga::make_plan(B, M, N, D, splits, &p);
    if (rc == MGA_OK) rc = mga::set_layout(&p, nullptr);
    if (rc == MGA_OK) rc = mga::check_call(q, k, v, o, p, ws, ws_bytes, true);
    if (rc != MGA_OK) return rc;
    if (B == 0 || M == 0) return MGA_OK;
    if (p.repack) {
        if (mga::launch_repack(p, k, ws, stream) != 0) return MGA_ERR_HIP;
        k = (const char *)ws + p.repack_off;
    }
    return mga::launch_partial(p, q, k, v, o, ws, stream) == 0 ? MGA_OK : MGA_ERR_HIP;
}

int mga_gqa_combine(void *o, int B, int M, int N, int D, int splits, const void *ws,
                    size_t ws_bytes, void *stream) {
    mga::Plan p;
    int rc = mga::make_plan(B, M, N, D, splits, &p);
    if (rc == MGA_OK) rc = mga::set_layout(&p, nullptr);
    if (rc == MGA_OK) rc = mga::check_call(nullptr, nullptr, nullptr, o, p, ws, ws_bytes, false);
    if (rc != MGA_OK) return rc;
    if (B == 0 || M == 0 || p.splits == 1) return MGA_OK;
    return mga::launch_combine(p, o, ws, stream) == 0 ? MGA_OK : MGA_ERR_HIP;
}

int mga_gqa_forward(const void *q, const void *k, const void *v, void *o, int B, int M, int N,
                    int D, int splits, void *ws, size_t ws_bytes, void *stream) {
    return mga_gqa_forward_strided(q, k, v, o, B, M, N, D, nullptr, splits, ws, ws_bytes, stream);
}

// The launches of one checked forward: K repack (if planned), partial
// kernel, combine (split plans), in that order on `stream`.
static int run_forward(const mga::Plan &p, const void *q, const void *k, const void *v, void *o, void *ws,
                       void *stream) {
    if (p.B == 0 || p.M == 0) return MGA_OK;
    if (p.repack) {
        if (mga::launch_repack(p, k, ws, stream) != 0) return MGA_ERR_HIP;
        k = (const char *)ws + p.repack_off;
    }
    if (mga::launch_partial(p, q, k, v, o, ws, stream) != 0) return MGA_ERR_HIP;
    if (p.splits > 1 && mga::launch_combine(p, o, ws, stream) != 0) return MGA_ERR_HIP;
    return MGA_OK;
}

int mga_gqa_forward_strided(const void *q, const void *k, const void *v, void *o, int B, int M,
                            int N, int D, const int64_t *strides, int splits, void *ws,
                            size_t ws_bytes, void *stream) {
    mga::Plan p;
    int rc = mga::make_plan(B, M, N, D, splits, &p);
    if (rc == MGA_OK) rc = mga::set_layout(&p, reinterpret_cast<const long long *>(strides));
    if (rc == MGA_OK) rc = mga::check_call(q, k, v, o, p, ws, ws_bytes, true);
    if (rc != MGA_OK) return rc;
    return run_forward(p, q, k, v, o, ws, stream);
}

int mga_gqa_forward_noalloc(const void *q, const void *k, const void *v, void *o, int B, int M,
                            int N, int D, const int64_t *strides, int splits, void *stream) {
    static_assert(mga::kScratchBytes == (size_t)MGA_NOALLOC_SCRATCH_BYTES, "scratch size in the header");
    mga::Plan p;
    int rc = mga::make_plan(B, M, N, D, splits, &p);
    if (rc == MGA_OK) rc = mga::set_layout(&p, reinterpret_cast<const long long *>(strides));
    if (rc != MGA_OK) return rc;
    if (p.ws_bytes > mga::kScratchBytes) return MGA_ERR_SCRATCH;
    void *ws = nullptr;
    if (p.ws_bytes > 0 && p.B > 0 && p.M > 0 && mga::scratch_ptr(&ws) != 0) return MGA_ERR_HIP;
    rc = mga::check_call(q, k, v, o, p, ws, mga::kScratchBytes, true);
    if (rc != MGA_OK) return rc;
    return run_forward(p, q, k, v, o, ws, stream);
}

int mga_gqa_plan(int B, int M, int N, int D, int splits, int *tile_rows, int *eff_splits) {
    mga::Plan p;
    const int rc = mga::make_plan(B, M, N, D, splits, &p);
    if (rc != MGA_OK) return rc;
    if (tile_rows) *tile_rows = p.tile_rows;
    if (eff_splits) *eff_splits = p.splits;
    return MGA_OK;
}

/* ---- QK-normalised variant ---- */

size_t mga_gqa_qknorm_workspace_bytes(int B, int M, int N, int D, int splits) {
    mga::Plan p;
    if (mga::make_plan(B, M, N, D, splits, &p, true) != MGA_OK) return 0;
    if (mga::set_layout(&p, nullptr) != MGA_OK) return 0;
    return p.ws_bytes;
}

int mga_gqa_qknorm_plan(int B, int M, int N, int D, int splits, int *tile_rows, int *eff_splits) {
    mga::Plan p;
    const int rc = mga::make_plan(B, M, N, D, splits, &p, true);
    if (rc != MGA_OK) return rc;
    if (tile_rows) *tile_rows = p.tile_rows;
    if (eff_splits) *eff_splits = p.splits;
    return MGA_OK;
}

int mga_gqa_qknorm_check_args(const void *q, const void *k, const void *v, const void *o, int B,
                              int M, int N, int D, float eps, const int64_t *strides, int splits,
                              const void *ws, size_t ws_bytes) {
    if (!(eps >= 0.f) || !std::isfinite(eps)) return MGA_ERR_INVALID_VALUE;
    mga::Plan p;
    int rc = mga::make_plan(B, M, N, D, splits, &p, true);
    if (rc == MGA_OK) rc = mga::set_layout(&p, reinterpret_cast<const long long *>(strides));
    if (rc != MGA_OK) return rc;
    return mga::check_call(q, k, v, o, p, ws, ws_bytes, true);
}

int mga_gqa_qknorm_forward(const void *q, const void *k, const void *v, void *o, int B, int M,
                           int N, int D, float eps, const int64_t *strides, int splits, void *ws,
                           size_t ws_bytes, void *stream) {
    int rc = mga_gqa_qknorm_check_args(q, k, v, o, B, M, N, D, eps, strides, splits, ws, ws_bytes);
    if (rc != MGA_OK) return rc;
    if (B == 0 || M == 0) return MGA_OK;
    mga::Plan p;
    mga::make_plan(B, M, N, D, splits, &p, true);
    mga::set_layout(&p, reinterpret_cast<const long long *>(strides));
    p.eps = eps;
    if (p.repack) {
        if (mga::launch_repack(p, k, ws, stream) != 0) return MGA_ERR_HIP;
        k = (const char *)ws + p.repack_off;
    }
    if (mga::launch_partial(p, q, k, v, o, ws, stream) != 0) return MGA_ERR_HIP;
    if (p.splits > 1 && mga::launch_combine(p, o, ws, stream) != 0) return MGA_ERR_HIP;
    return MGA_OK;
}

}  // extern "C"
