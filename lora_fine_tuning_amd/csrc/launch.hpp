// Internal interface between the C-ABI layer (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include "lora_fused.h"

namespace lora {

struct ChunkEntry;

// Rows handled by one work item of each low-rank kernel.
constexpr int kF1Rows = 64;    // mask + down-projection
constexpr int kBwdRows = 256;  // dS/dB and dA kernels
constexpr int kF1KSub = 128;   // k columns per staged slice of A in F1

// The streaming low-rank kernels work on ranks in tiles of up to 32; ranks
// above 32 take ceil(r/32) tiles of 32 (one launch, one tile per grid slice).
inline int rank_tiles(int r_lds) { return r_lds > 32 ? (r_lds + 31) / 32 : 1; }

// F1's streaming form (each work-group covers all of k, no partial sums)
// serves ranks up to 128; its 32-bit buffer offsets need 64*k < 2^31.
inline bool f1_streaming(int r_lds, int64_t k) { return r_lds <= 128 && k * 64 < (int64_t(1) << 31); }
// The single-adapter streaming F1 takes rank tiles of 64 when the rank spans an
// even number of 32-rank tiles (33..64, 97..128).
inline bool f1_rank64(int r_lds, bool multi) {
    return !multi && r_lds > 32 && r_lds <= 128 && ((r_lds + 31) / 32) % 2 == 0;
}

// Rows per B2 work item (the dA partials are one per item): 256, or taller
// when the grid (items x 256-column tiles of k x rank tiles) would still have
// about 512 work-groups -- fewer partials for wide k or many rank tiles -- or
// when the partials would otherwise rival X in bytes (high ranks).
inline int b2_rows(int64_t m, int64_t k, int r_lds) {
    const int rt = r_lds > 128 ? (r_lds + 31) / 32 : 1;
    const int64_t want = m * ((k + 255) / 256) * rt / 512;
    int64_t rows = std::max<int64_t>(kBwdRows, (want + 31) / 32 * 32);
    if (r_lds <= 128) {
        // the single-pass form's dA partials (a k x RP block per item) stay at
        // most a quarter of the item's X bytes (rows >= 8 RP) while the grid
        // keeps at least 256 work-groups
        const int nb = (r_lds + 15) / 16;
        const int64_t rp = 16 * (nb <= 1 ? 1 : nb <= 2 ? 2 : nb <= 4 ? 4 : 8);
        const int64_t wg_cap = std::max<int64_t>(kBwdRows, m * ((k + 255) / 256) / 256 / 32 * 32);
        rows = std::max<int64_t>(rows, std::min<int64_t>(8 * rp, wg_cap));
    }
    rows = std::min<int64_t>(rows, std::max<int64_t>(kBwdRows, (m + 31) / 32 * 32));
    // the kernels address an item's rows of X with 32-bit offsets
    const int64_t cap = ((int64_t(1) << 31) - 1) / (2 * std::max<int64_t>(k, 1)) / 32 * 32;
    return (int)std::max<int64_t>(std::min<int64_t>(rows, cap), std::min<int64_t>(kBwdRows, cap));
}

// B1 / B2 streaming forms: ranks up to 32, or up to 128 in rank tiles when
// the S / dS row stride is a multiple of 4 floats (16-byte row pieces).
inline bool bwd_streaming(int r_lds, int RS) { return r_lds <= 32 || (r_lds <= 128 && RS % 4 == 0); }

// Kernel timing hooks (api.cpp).  prof_begin returns a slot or -1.
int prof_begin(const char *name, hipStream_t stream);
void prof_end(int slot, hipStream_t stream);

// Adapter source for the launchers: either one adapter given by value or a
// device table plus chunk tables built by the router.
struct AdapterSource {
    // single adapter
    const void *A;
    const void *B;
    void *dA;
    void *dB;
    int32_t r;
    float alpha;
    float p;
    // multi adapter (table != nullptr)
    const lora_adapter *table;
    int32_t num_adapters;
    int32_t r_cap;
    const int64_t *seg_off;
    const int32_t *seg_adapter;
    int32_t num_segments;
    // chunk tables (multi only)
    const ChunkEntry *chunks_f1;
    const int32_t *count_f1;
    const ChunkEntry *chunks_bwd;
    const int32_t *count_bwd;
    const ChunkEntry *chunks_b1;
    const int32_t *count_b1;
};

// Which router table a kernel's work items come from.
enum WorkTable { kTabF1 = 0, kTabBwd = 1, kTabB1 = 2 };

// ad_items (may be NULL): work items of each adapter in the backward table.
hipError_t launch_router(const int64_t *seg_off, const int32_t *seg_adapter, int nseg, int m,
                         const lora_adapter *adapters, int nad, int r_cap, ChunkEntry *t_f1,
                         int32_t *c_f1, int cap_f1, ChunkEntry *t_bwd, int32_t *c_bwd, int rows_bwd, int cap_bwd,
                         ChunkEntry *t_b1, int32_t *c_b1, int rows_b1, int cap_b1, hipStream_t stream,
                         int32_t *ad_items = nullptr);

// s2 (streaming form only; may be NULL): also write alpha*S split into bf16
// [hi | lo] rows of 2*s2_rp columns for the forward GEMM's extra K columns.
hipError_t launch_f1(const void *X, int m, int k, const AdapterSource &src, int chunk_cap,
                     uint64_t seed, uint64_t offset, uint32_t *keep_bits, float *out, int RS,
                     int KS, int ksl, hipStream_t stream, uint16_t *s2 = nullptr, int s2_rp = 0);

// F1 for 32 < r_lds <= 128: 64-row chunks sharing A, k in KS slices of ksl
// columns (multiples of 128); with KS > 1 the slices' partials ([KS][m][16 *
// f1w_blocks] fp32) are added by a second launch, which also writes the
// forward GEMM's split of alpha*S when s2 is given.
inline int f1w_blocks(int r_lds) { return r_lds <= 64 ? 4 : 8; }
inline bool f1w_ok(int r_lds, int64_t k) { return r_lds > 32 && r_lds <= 128 && k * 64 < (int64_t(1) << 31); }
hipError_t launch_f1w(const void *X, int m, int k, const AdapterSource &src, int chunk_cap, uint64_t seed,
                      uint64_t offset, uint32_t *keep_bits, float *S, int RS, float *part, int KS, int ksl,
                      hipStream_t stream, uint16_t *s2 = nullptr, int s2_rp = 0);

hipError_t launch_sum_partials(const float *part, int nparts, size_t part_stride, size_t count,
                               float *out, const char *name, hipStream_t stream);

// Launch shape of B1 (dS and dB partials).  Work-groups cover C1 columns of
// a row group: `rows` rows of the single adapter, or one router chunk of the
// mixed-adapter form.  dS gets one partial per column tile (CT), dB one per
// row group (slots).  The streaming kernel serves ranks up to 32; its 32-bit
// direct-to-LDS offsets need rows * n * 2 < 2^31.
struct B1Shape {
    bool streaming;
    int cw;  // streaming: C1 = 256 * cw
    int C1, CT, rows, slots;
};
inline B1Shape b1_shape(int64_t m, int64_t n, int r_lds, int RS, bool multi, int nseg) {
    B1Shape s{};
    const int64_t maxrows = ((int64_t(1) << 31) - 1) / (2 * n) / 32 * 32;
    s.streaming = bwd_streaming(r_lds, RS) && maxrows >= 32;
    if (!s.streaming) {
        s.cw = 1;
        s.C1 = r_lds <= 128 ? 256 : 128;
        s.CT = (int)((n + s.C1 - 1) / s.C1);
        s.rows = kBwdRows;
    } else {
        // 256-column tiles: two work-groups share a CU (measured faster than
        // 512-column tiles at one per CU, despite twice the dS partials)
        s.cw = 1;
        s.C1 = 256 * s.cw;
        s.CT = (int)((n + s.C1 - 1) / s.C1);
        // about 512 work-groups; fewer, taller row groups mean fewer dB partials
        int64_t nrg = std::max<int64_t>(1, 512 / s.CT);
        nrg = std::min<int64_t>(nrg, std::max<int64_t>(1, (m + 31) / 32));
        int64_t rows = std::max<int64_t>(32, 32 * (((m + nrg - 1) / nrg + 31) / 32));
        // a row group's dB partial (r x n fp32) at most half the bytes of its
        // dY rows: rows >= 4 r
        rows = std::max<int64_t>(rows, 32 * ((4 * (int64_t)r_lds + 31) / 32));
        s.rows = (int)std::min(rows, maxrows);
    }
    // mixed adapters: the router cuts each segment into runs of `rows`
    s.slots = (int)((m + s.rows - 1) / s.rows) + (multi ? nseg : 0);
    return s;
}

hipError_t launch_b1(const void *dY, const float *S, int m, int n, int RS, const AdapterSource &src,
                     const B1Shape &sh, float *dSpart, float *dBpart, hipStream_t stream);

hipError_t launch_b2(const void *X, const uint32_t *keep, const float *dS, int m, int k, int RS, int rows,
                     const AdapterSource &src, int chunk_cap, int C2, float *dApart,
                     hipStream_t stream);

// which = 0: dB (r x n per adapter from [chunk][RS][n]); 1: dA (k x r from [chunk][k][RS]).
// dS = fixed-order sum of B1's nparts column-tile partials (skipped when
// nparts == 1) and dB = per-adapter sum of its row-group partials, one launch.
// dss (optional): also write rows of [hi | lo] bf16 of s*dS for the dA pass
// and the dX epilogue, dss_ld (presplit_ld) bf16 apart
hipError_t launch_b1_reduce(const float *dSpart, int nparts, float *dS, const float *dBpart, int m, int n,
                            int RS, const AdapterSource &src, int rows, int slots, hipStream_t stream,
                            uint16_t *dss = nullptr, int dss_ld = 0);

// The single-pass dA kernel (ranks up to 128 in one pass over X) serves
// r_lds <= 128 when S / dS rows are 16-byte pieces (RS % 4 == 0).  Its
// partials are [item][ceil(k/256)][256][16 * b2w_blocks] fp32; a second
// launch adds each adapter's partials in item order and writes dA.
inline int b2w_blocks(int r_lds) {
    const int nb = (r_lds + 15) / 16;
    return nb <= 1 ? 1 : nb <= 2 ? 2 : nb <= 4 ? 4 : 8;
}
inline bool b2w_ok(int r_lds, int RS) { return r_lds <= 128 && RS % 4 == 0; }
// items: grid rows of work items (single: ceil(m / rows); multi: the
// backward table's capacity); ad_items: multi only (the router's
// per-adapter counts).
// Row stride (bf16) of the split s*dS rows the dA pass needs above 32 ranks
// (0: the pass splits dS itself)
inline int presplit_ld(int r_lds) { return b2w_ok(r_lds, 4) && b2w_blocks(r_lds) >= 4 ? 32 * b2w_blocks(r_lds) : 0; }
hipError_t launch_b2w(const void *X, const uint32_t *keep, const float *dS, int m, int k, int RS, int rows,
                      const AdapterSource &src, int items, float *part, const int32_t *ad_items,
                      hipStream_t stream, const uint16_t *dss = nullptr, int dss_ld = 0);

// rows: rows per partial of the single-adapter form; slots: partials
// written (an upper bound in the mixed-adapter form, where the router's chunk
// count decides).
hipError_t launch_grad_reduce(int which, const float *part, int m, int k, int n, int RS,
                              const AdapterSource &src, int rows, int slots, hipStream_t stream);

hipError_t launch_mask(uint64_t seed, uint64_t offset, int m, int k, float p, uint32_t *bits,
                       hipStream_t stream);

// GEMM: C = Arow * op(Bcol) (+ LoRA term).  nn: Bcol is K x N (W of the
// forward); otherwise Bcol is N x K (W seen transposed by the backward).
// epi 0: none; 1: + alpha*S*B (F2); 2: + s*keep.(dS A^T) (B3).
hipError_t launch_gemm(bool nn, int epi, const void *Arow, const void *Bcol, void *C, int M, int N,
                       int K, const float *Sx, int RS, const uint32_t *keep, int KW,
                       const AdapterSource &src, hipStream_t stream, const uint16_t *dss = nullptr,
                       int dss_ld = 0);

// Forward GEMM with the LoRA term as kx extra K columns: Y = [X | S2] [W ; B' ]
// where S2 holds alpha*S split into bf16 hi and lo parts of kx/2 ranks each and
// B' repeats B's rows for both halves (rows past r zero).  B must be 16-byte
// aligned (N is a multiple of 8).
// Forward at p = 0 with [W | A] as one operand: Y = X W + alpha (X A) B and
// S = X A (fp32, M x r), r 8 or 16, A / B / S 16-byte aligned.
hipError_t launch_gemm_cat(const void *X, const void *W, const void *A, const void *B, void *Y, float *S,
                           int M, int N, int K, int r, float alpha, hipStream_t stream);
hipError_t launch_gemm_kext(const void *X, const void *W, void *Y, int M, int N, int K, const uint16_t *S2,
                            int kx, const void *B, int r, hipStream_t stream);

size_t gemm_lds_bytes();

// DoRA norm of W + alpha A B per output feature (column): splits of W's rows
// (multiples of 32) so that about 512 work-groups of 256 columns run (two per
// CU), or above rank 128, where one work-group fills a CU, DORA_WGS_BIG; each
// split's rows * n * 2 bytes under 2^31.
struct DoraPlan {
    int splits, rows;
};
constexpr int64_t DORA_WGS_BIG = 256;
inline DoraPlan dora_plan(int64_t k, int64_t n, int r) {
    const int64_t ctiles = (n + 255) / 256;
    const int64_t maxrows = std::max<int64_t>(32, ((int64_t(1) << 31) - 1) / (2 * n) / 32 * 32);
    const int64_t wgs = r > 128 ? DORA_WGS_BIG : 512;
    int64_t splits = std::max<int64_t>(1, std::min<int64_t>((wgs + ctiles - 1) / ctiles, (k + 255) / 256));
    int64_t rows = 32 * (((k + splits - 1) / splits + 31) / 32);
    rows = std::min(rows, maxrows);
    splits = (k + rows - 1) / rows;
    return DoraPlan{(int)splits, (int)rows};
}
hipError_t launch_dora_norm(const void *W, const void *A, const void *B, int k, int n, int r, float alpha,
                            const DoraPlan &pl, float *part, float *norm, hipStream_t stream);

}  // namespace lora
