// DoRA's norm of the adapted weight, one value per output feature:
//   norm[j] = || W[:, j] + alpha * (A B)[:, j] ||_2,  W k x n, A k x r, B r x n.
// (DoRA reading of a "row norm" of W + sBA in the out x in convention of the
// page on the factored DoRA norm -- "core method"; here X W with W k x n, so
// an output feature is a column.)  The page splits the squared norm into a
// base, a cross and a Gram term so the dense product is never materialised.
// On gfx950 the pass over W is HBM-bound with room to spare on the matrix
// cores (2r flops per 2-byte element of W, below the machine balance for every
// rank up to 256), so each 32-row x 256-column tile of W gets its A B tile
// from MFMA in registers and the squares of W + alpha A B are summed directly:
// nothing dense is stored and no cancellation between the three terms occurs.
//
// Work-group = a range of W's rows (a split) x 256 columns; four waves of 64
// columns each, or for ranks above 128 eight waves, two per 64 columns, each
// taking one 16-row half of every 32-row sub-block.  W's rows stream through a
// 3-stage ring of direct-to-LDS loads (with A's matching rows); B's fragments
// for the work-group's columns are loaded once.  Each split writes per-column
// partial sums of squares; a second kernel adds the splits in a fixed order and
// takes the square root.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace lora {

namespace {

struct DoraParams {
    const uint16_t *W, *A, *B;
    int k, n, r;
    float alpha;
    int rows;     // W rows per split (a multiple of 32)
    float *part;  // [split][n] partial sums of squares
};

constexpr int DORA_SUB = 32 * 512;  // one 32-row x 256-column bf16 tile
constexpr int DORA_NST_BIG = 3;  // ring stages above rank 128
constexpr int dora_nst(int rpq) { return rpq == 8 ? DORA_NST_BIG : 3; }

// Waves per work-group.  Above rank 128 B's staging fills a CU's LDS, so one
// work-group runs per CU; eight waves then put two on each SIMD, and one
// wave's matrix work overlaps the other's LDS reads and waits.
constexpr int dora_nw(int rpq) { return rpq == 8 ? 8 : 4; }
constexpr int dora_nai(int rpq) { return rpq <= 2 ? 1 : rpq / 2; }  // 1 KiB A loads per stage, per 4 waves
constexpr int dora_stage(int rpq) { return DORA_SUB + 4 * dora_nai(rpq) * 1024; }
// LDS: for r <= 32 B's one chunk sits past the ring, so both load together
// (two work-groups still share a CU); larger ranks stage all of B's 32-rank
// chunks in the space the ring uses afterwards
constexpr bool dora_b_apart(int rpq) { return rpq == 1; }
constexpr int dora_b_off(int rpq) { return dora_b_apart(rpq) ? dora_nst(rpq) * dora_stage(rpq) : 0; }
constexpr int dora_lds(int rpq) {
    // (eight waves: 1 KiB past the ring for the half sums)
    return dora_b_apart(rpq) ? dora_nst(rpq) * dora_stage(rpq) + DORA_SUB
         : (dora_nst(rpq) * dora_stage(rpq) + (dora_nw(rpq) == 8 ? 1024 : 0) > rpq * DORA_SUB
                ? dora_nst(rpq) * dora_stage(rpq) + (dora_nw(rpq) == 8 ? 1024 : 0)
                : rpq * DORA_SUB);
}

// Half of tile_rows8: rows row0 .. row0+3 (row0 % 4 == 0) of column
// 16*cb + (lane % 16), 4 bf16 per lane.
__device__ __forceinline__ uint2 tile_rows4(const lds_char *tile, int row0, int cb, int lane) {
    const int a = lane & 15;
    return lds_read_tr4(tile + swz512_off(row0 + (a >> 2), 2 * cb + ((a & 3) >> 1)) + (a & 1) * 8);
}

// RPQ: rank steps of 32 (ceil(r / 32)); AVEC: r % 8 == 0 (16-byte A reads)
template <int RPQ, bool AVEC>
__global__ __launch_bounds__(64 * dora_nw(RPQ)) void dora_norm_kernel(DoraParams P) {
    constexpr int NW = dora_nw(RPQ);
    constexpr int NH = 8 / NW;               // 16-row halves per wave
    constexpr int NJ = 16 / NW;              // 1 KiB W (and B) loads per wave per stage
    constexpr int NAI = dora_nai(RPQ) * 4 / NW;
    constexpr int STAGE = dora_stage(RPQ);
    constexpr int DORA_NST = dora_nst(RPQ);
    // A's rows go through LDS only when r % 8 == 0: then every 16-byte piece of
    // a sub-block's A image lies wholly inside A (a piece straddling A's end
    // would read as zero); otherwise A's elements are read from global memory
    constexpr int NDMA = NJ + (AVEC ? NAI : 0);  // direct-to-LDS loads per wave per stage
    extern __shared__ uint4 dora_smem[];
    lds_char *smem = (lds_char *)dora_smem;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cw = wave & 3;   // the wave's 64 columns
    const int hw = wave >> 2;  // its half when NH == 1
    const int g = lane >> 4, li = lane & 15;
    const int r = P.r;
    const int row_lo = (int)blockIdx.x * P.rows;
    const int nrows = min(P.k, row_lo + P.rows) - row_lo;  // >= 1: the host sizes the splits
    const int nsb = (nrows + 31) / 32;
    const int n0 = (int)blockIdx.y * 256;

    // host guarantees nrows * n * 2 < 2^31 and (r + 32) * n * 2 < 2^31; rows
    // past a descriptor's end read as zero
    const sgpr4_t dW = make_desc(P.W + (size_t)row_lo * P.n, (uint32_t)((uint64_t)nrows * P.n * 2));
    const sgpr4_t dB = make_desc(P.B, (uint32_t)((uint64_t)r * P.n * 2));
    const sgpr4_t dA = make_desc(P.A + (size_t)row_lo * r, (uint32_t)((uint64_t)nrows * r * 2));
    const uint32_t asb = 32u * (uint32_t)r * 2u;  // A bytes of one 32-row sub-block

    // tile loads: instruction j of wave w fills LDS rows 2(NJ w + j), +1 (512 B
    // each); LDS chunk (lane & 31) of row rr holds global chunk (lane & 31) ^ swz512(rr)
    uint32_t offT[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int rr = 2 * (NJ * wave + j) + (lane >> 5);
        const int col = n0 + 8 * ((lane & 31) ^ swz512(rr));
        offT[j] = col < P.n ? (uint32_t)(rr * P.n + col) * 2u : kOOBL;
    }
    // A's 32 rows of a sub-block as one image with row stride 2r bytes (bytes
    // past the sub-block read as zero).  When a row holds a power-of-two
    // number RC >= 8 of 16-byte chunks, chunk c of image row i holds A's chunk
    // c ^ aswz(i), so the 16 rows one fragment read touches fall in different
    // banks (they sit 2r bytes apart, a multiple of the bank period).
    const int RC = r / 8;
    const int aswz_mask = (AVEC && RC >= 8 && (RC & (RC - 1)) == 0) ? min(RC, 16) - 1 : 0;
    auto aswz = [&](int i) { return ((i & 3) | ((i >> 3) << 2)) & aswz_mask; };
    uint32_t offA[NAI];  // image byte -> sub-block byte of A, per load (kOOBL past the image)
#pragma unroll
    for (int q = 0; q < NAI; ++q) {
        const uint32_t b = (uint32_t)(NW * q + wave) * 1024u + (uint32_t)lane * 16u;
        if (!AVEC || b >= asb) {
            offA[q] = kOOBL;
        } else {
            const int ci = (int)(b >> 4), i = ci / RC, c = ci % RC;
            offA[q] = (uint32_t)(i * RC + (c ^ aswz(i))) * 16u;
        }
    }
    // sub-block sb: its W tile, then A's image
    auto issue = [&](int sb, int stage) {
        const uint32_t base = lds0 + stage * STAGE;
        const bool live = sb < nsb;
        const uint32_t wo = live ? (uint32_t)sb * 32u * (uint32_t)P.n * 2u : 0u;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            dma16(dW, (!live || offT[j] == kOOBL) ? kOOBL : offT[j] + wo, base + (NJ * wave + j) * 1024);
        if constexpr (AVEC) {
#pragma unroll
            for (int q = 0; q < NAI; ++q)
                dma16(dA, (live && offA[q] != kOOBL) ? (uint32_t)sb * asb + offA[q] : kOOBL,
                      base + DORA_SUB + (uint32_t)(NW * q + wave) * 1024u);
        }
    };
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(P.A + (size_t)row_lo * r, (uint64_t)nrows * r * 2);

    // B fragments (MFMA column operand): ranks 32q + 8g .. +7 of column
    // n0 + 64 cw + 16b + li; all 32-rank chunks land in LDS together (chunk q
    // at q * 16 KiB), then the ring reuses the space
    constexpr int BOFF = dora_b_off(RPQ);
    uint4 bfr[RPQ][4];
#pragma unroll
    for (int q = 0; q < RPQ; ++q) {
        const uint32_t bo = (uint32_t)q * 32u * (uint32_t)P.n * 2u;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            dma16(dB, offT[j] == kOOBL ? kOOBL : offT[j] + bo, lds0 + BOFF + q * DORA_SUB + (NJ * wave + j) * 1024);
    }
    if constexpr (dora_b_apart(RPQ)) {
#pragma unroll
        for (int q = 0; q < DORA_NST - 1; ++q) issue(q, q);
        wait_vmcnt<NDMA * (DORA_NST - 1)>();  // B has landed (issued first)
    } else {
        wait_vmcnt<0>();
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < RPQ; ++q)
#pragma unroll
        for (int b = 0; b < 4; ++b) bfr[q][b] = tile_rows8(smem + BOFF + q * DORA_SUB, 8 * g, 4 * cw + b, lane);
    if constexpr (!dora_b_apart(RPQ)) __syncthreads();  // the ring rewrites the space

    // The A B tile of a 16-row half h comes from MFMA with row i' = 4c + v
    // standing for W row 8c + 4h + v: then the MFMA result of lane (c, li),
    // register v, pairs with the W values the transposing read of rows
    // 8c .. 8c+7 hands the same lane (half 0 the first four, half 1 the rest).
    const int arow0 = 8 * (li >> 2) + (li & 3);
    auto a_frag = [&](const lds_char *at, int sb, int h, int q) -> uint4 {
        const int t0 = 32 * q + 8 * g, arow = arow0 + 4 * h;
        if constexpr (AVEC) {
            const uint4 v = *(const uint4 *)(at + arow * r * 2 + (((t0 >> 3) ^ aswz(arow)) << 4));
            return t0 < r ? v : make_uint4(0u, 0u, 0u, 0u);
        } else {
            // element (row, t) of the split at byte 2 (row r + t); rows past the
            // split read as zero
            const uint32_t e0 = (uint32_t)((32 * sb + arow) * r + t0) * 2u;
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = t0 + 2 * e < r
                    ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rA, e0 + 4u * e, 0, 0) : 0u;
                const uint32_t hi = t0 + 2 * e + 1 < r
                    ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rA, e0 + 4u * e + 2u, 0, 0) : 0u;
                w[e] = lo | (hi << 16);
            }
            return make_uint4(w[0], w[1], w[2], w[3]);
        }
    };

    float sq[4] = {0.f, 0.f, 0.f, 0.f};
    const float alpha = P.alpha;
    if constexpr (!dora_b_apart(RPQ)) {
#pragma unroll
        for (int q = 0; q < DORA_NST - 1; ++q) issue(q, q);
    }
    wait_vmcnt<NDMA * (DORA_NST - 2)>();
    __syncthreads();
    int stage = 0, lstage = DORA_NST - 1;
    for (int sb = 0; sb < nsb; ++sb) {
        issue(sb + DORA_NST - 1, lstage);
        const lds_char *wt = smem + stage * STAGE;
        const lds_char *at = wt + DORA_SUB;
        uint4 afr[NH][RPQ];
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int q = 0; q < RPQ; ++q) afr[h][q] = a_frag(at, sb, NH == 2 ? h : hw, q);
        // 4 NH independent accumulation chains (4 column blocks x the wave's halves)
        f32x4_t d[NH][4];
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
            for (int b = 0; b < 4; ++b) d[h][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < RPQ; ++q)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int h = 0; h < NH; ++h) d[h][b] = mfma16x16x32(afr[h][q], bfr[q][b], d[h][b]);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            // W rows 8c + 4h + v of the lane's column, two to a word
            uint32_t wh[2 * NH];
            if constexpr (NH == 2) {
                const uint4 wv = tile_rows8(wt, 8 * g, 4 * cw + b, lane);
                wh[0] = wv.x, wh[1] = wv.y, wh[2] = wv.z, wh[3] = wv.w;
            } else {
                const uint2 wv = tile_rows4(wt, 8 * g + 4 * hw, 4 * cw + b, lane);
                wh[0] = wv.x, wh[1] = wv.y;
            }
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint32_t wb = v & 1 ? wh[2 * h + (v >> 1)] >> 16 : wh[2 * h + (v >> 1)] & 0xFFFFu;
                    const float x = bf16_to_f32(wb) + alpha * d[h][b][v];
                    sq[b] += x * x;
                }
        }
        wait_vmcnt<NDMA * (DORA_NST - 2)>();
        __syncthreads();
        stage = stage == DORA_NST - 1 ? 0 : stage + 1;
        lstage = lstage == DORA_NST - 1 ? 0 : lstage + 1;
    }
    wait_vmcnt<0>();

    // the four lane groups hold disjoint rows of the same column; with one
    // half per wave, the second half's sums pass through LDS past the ring
    // (the loop's last barrier follows every wave's last read of the ring,
    // and the space past it held only B)
    float s[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        s[b] = sq[b];
        s[b] += __shfl_xor(s[b], 16);
        s[b] += __shfl_xor(s[b], 32);
    }
    if constexpr (NH == 1) {
        static_assert(dora_lds(RPQ) >= DORA_NST * STAGE + 1024, "no room for the half sums");
        float *hs = (float *)(smem + DORA_NST * STAGE);
        if (hw == 1 && g == 0) {
#pragma unroll
            for (int b = 0; b < 4; ++b) hs[64 * cw + 16 * b + li] = s[b];
        }
        __syncthreads();
        if (hw == 1) return;
#pragma unroll
        for (int b = 0; b < 4; ++b) s[b] += hs[64 * cw + 16 * b + li];
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int col = n0 + 64 * cw + 16 * b + li;
        if (g == 0 && col < P.n) P.part[(size_t)blockIdx.x * P.n + col] = s[b];
    }
}

// norm[j] = sqrt of the splits' partial sums, added in split order
__global__ __launch_bounds__(256) void dora_finish_kernel(const float *part, int splits, int n, float *norm) {
    const int j = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (j >= n) return;
    float s = 0.f;
    for (int sp = 0; sp < splits; ++sp) s += part[(size_t)sp * n + j];
    norm[j] = sqrtf(s);
}

template <int RPQ, bool AVEC>
void launch_dora_t(const DoraParams &P, dim3 grid, hipStream_t stream) {
    constexpr size_t lds = (size_t)dora_lds(RPQ);
    if (lds > 64 * 1024)
        (void)hipFuncSetAttribute((const void *)dora_norm_kernel<RPQ, AVEC>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((dora_norm_kernel<RPQ, AVEC>), grid, dim3(64 * dora_nw(RPQ)), lds, stream, P);
}

}  // namespace

hipError_t launch_dora_norm(const void *W, const void *A, const void *B, int k, int n, int r, float alpha,
                            const DoraPlan &pl, float *part, float *norm, hipStream_t stream) {
    DoraParams P;
    P.W = (const uint16_t *)W;
    P.A = (const uint16_t *)A;
    P.B = (const uint16_t *)B;
    P.k = k;
    P.n = n;
    P.r = r;
    P.alpha = alpha;
    P.rows = pl.rows;
    P.part = part;
    const dim3 grid((unsigned)pl.splits, (unsigned)((n + 255) / 256));
    const bool avec = r % 8 == 0;
    int slot = prof_begin("dora_norm_pass", stream);
    if (r <= 32) avec ? launch_dora_t<1, true>(P, grid, stream) : launch_dora_t<1, false>(P, grid, stream);
    else if (r <= 64) avec ? launch_dora_t<2, true>(P, grid, stream) : launch_dora_t<2, false>(P, grid, stream);
    else if (r <= 128) avec ? launch_dora_t<4, true>(P, grid, stream) : launch_dora_t<4, false>(P, grid, stream);
    else avec ? launch_dora_t<8, true>(P, grid, stream) : launch_dora_t<8, false>(P, grid, stream);
    prof_end(slot, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    slot = prof_begin("dora_norm_finish", stream);
    hipLaunchKernelGGL(dora_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, part,
                       pl.splits, n, norm);
    prof_end(slot, stream);
    return hipGetLastError();
}

}  // namespace lora
