// MFMA bf16 GEMM of the gfx950 LoRA path, with the LoRA branch fused into its
// epilogue so the full-size output is written once:
//   F2  (nn, epi 1): Y  = X W + alpha * S B            (juhe.plus blog on
//        LoRAFusion, section 4.1, forward item 2: the frozen GEMM and the
//        alpha*S*B up-projection accumulate into the same output)
//   B3  (nt, epi 2): dX = dY W^T + s * keep.(dS A^T)   (same section, backward
//        item 5: the base gradient and the LoRA path share one pass, so no
//        partial input gradient is re-read or re-written)
//   frozen (epi 0):  Y = X W and dX = dY W^T, the baseline layer.
//
// Tiling: 256 x 256 output tile per work-group of 4 waves (2 x 2), 64-deep K
// steps through double-buffered LDS (2 x 72 KiB), v_mfma_f32_32x32x16_bf16
// with fp32 accumulators (each wave a 4 x 4 grid of 32 x 32 tiles).  The
// column-side operand is the MFMA's first source so every lane ends up with 4
// consecutive output columns of one row (8-byte stores).  For the forward W is
// k x n (n contiguous): each thread loads an 8 x 8 block and transposes it in
// registers so the LDS copy is K-contiguous.  Work-group ids are remapped so
// each XCD gets a contiguous range of tiles, visited in groups of 8 row panels.
//
// The LoRA terms run after the K loop as extra rank-deep MFMA steps whose
// operands come straight from global memory: fp32 S (or dS) as hi+lo bf16
// pairs times B (or A).  For the masked backward term the rank-deep product
// goes to a second accumulator, one 32-row band at a time, and is added under
// the stored keep bits.  Mixed-adapter tiles run one such pass per segment
// overlapping the tile (rows of other segments contribute zero).
#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"

namespace lora {

constexpr int GBM = 256, GBN = 256;

struct GemmParams {
    const uint16_t *Arow;  // M x K
    const uint16_t *Bcol;  // nn: K x N; nt: N x K
    uint16_t *C;           // M x N
    int M, N, K;
    int tiles_m, tiles_n;
    const float *Sx;  // S (epi 1) or dS (epi 2), M x RS
    int RS;
    const uint32_t *keep;  // epi 2 (nullptr = all kept)
    int KW;
    // single adapter: ext = B (epi 1, r x N) or A (epi 2, N x r)
    const uint16_t *ext;
    int ext_r;
    float ext_scale;  // alpha (epi 1) or s (epi 2); multi: from p / alpha per adapter
    // multi adapter
    const lora_adapter *adapters;
    int num_adapters, r_cap;
    const int64_t *seg_off;
    const int32_t *seg_adapter;
    int nseg;
};

__device__ __forceinline__ void tile_coords(int wg, int G, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int xcd = wg & 7, local = wg >> 3, per = G >> 3, rem = G & 7;
    const int lid = xcd * per + min(xcd, rem) + local;
    constexpr int GROUP = 8;
    const int width = GROUP * tiles_n;
    const int group = lid / width, first = group * GROUP;
    const int gsz = min(tiles_m - first, GROUP);
    const int in = lid - group * width;
    tm = first + in % gsz;
    tn = in / gsz;
}

// One item of the LoRA epilogue: rows [lo, hi) with one adapter.
struct ExtItem {
    int lo, hi;
    const uint16_t *w;  // B (r x N) or A (N x r)
    int r;
    float scale;
};

// Rank-deep MFMA step inputs for one 32-row band: fp32 rows of S/dS times
// `scale`, split into hi/lo fragments; rows outside [lo, hi) give zero.
__device__ __forceinline__ void row_ext_frags(const GemmParams &P, const ExtItem &it, int row, int rr0,
                                              int lane, uint4 &hi, uint4 &lo) {
    float v[8];
    const bool ok = row >= it.lo && row < it.hi;
    const float *src = P.Sx + (size_t)(ok ? row : 0) * P.RS;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int rr = rr0 + 8 * (lane >> 5) + e;
        v[e] = (ok && rr < it.r) ? it.scale * src[rr] : 0.f;
    }
    split_frag(v, hi, lo);
}

// Column-side fragment of the rank-deep step: 8 consecutive ranks of output
// column `col`.  epi 1 reads B[rr][col] (stride N); epi 2 reads A[col][rr].
template <int EPI>
__device__ __forceinline__ uint4 col_ext_frag(const GemmParams &P, const ExtItem &it, int col, int rr0,
                                              int lane) {
    uint32_t h[8];
    const bool cok = col < P.N;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int rr = rr0 + 8 * (lane >> 5) + e;
        uint32_t x = 0;
        if (cok && rr < it.r) x = EPI == 1 ? it.w[(size_t)rr * P.N + col] : it.w[(size_t)col * it.r + rr];
        h[e] = x;
    }
    return make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
}

template <int EPI, bool MULTI>
__device__ __forceinline__ bool get_item(const GemmParams &P, int s, ExtItem &it) {
    if (!MULTI) {
        it.lo = 0;
        it.hi = P.M;
        it.w = P.ext;
        it.r = P.ext_r;
        it.scale = P.ext_scale;
        return true;
    }
    const int64_t o0 = P.seg_off[s], o1 = P.seg_off[s + 1];
    it.lo = (int)max((int64_t)0, min(o0, (int64_t)P.M));
    it.hi = (int)max((int64_t)it.lo, min(o1, (int64_t)P.M));
    const int a = P.seg_adapter[s];
    if (a < 0 || a >= P.num_adapters || it.hi <= it.lo) return false;
    const lora_adapter ad = P.adapters[a];
    if (ad.r < 1 || ad.r > P.r_cap) return false;
    it.r = ad.r;
    it.w = (const uint16_t *)(EPI == 1 ? ad.B : ad.A);
    it.scale = EPI == 1 ? ad.alpha : drop_scale(ad.p);
    return true;
}

// First segment whose end is beyond row m0 (segments sorted by offset).
__device__ __forceinline__ int first_segment(const GemmParams &P, int m0) {
    int lo = 0, hi = P.nseg;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (P.seg_off[mid + 1] <= (int64_t)m0) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

// Buffer resource over `bytes` bytes from `base`; loads past the end return 0
// and stores past the end are dropped, so edge tiles need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint64_t bytes) {
    const uint32_t nrec = (uint32_t)(bytes < 0x7FFFFFF0ull ? bytes : 0x7FFFFFF0ull);
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)nrec, 0x00020000);
}
constexpr uint32_t kOOB = 0x80000000u;  // an offset beyond every resource

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

constexpr int BK = 64;              // K depth of one LDS stage
constexpr int NST = 2;              // stages in the LDS ring
constexpr int ROWB = BK * 2;        // bytes per LDS row of a K-contiguous tile
constexpr int CPR = BK / 8;         // 16-byte chunks per such row
constexpr int TILE_BYTES = GBM * ROWB;  // one operand tile (the NN W tile is BK x 512 B, same size)
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr int LPW = BK / 8;         // 1-KiB direct-to-LDS loads per wave per operand per stage
// XOR swizzle of 16-byte chunks: conflict-free 16-lane b128 reads of 16
// consecutive rows (K-contiguous tiles) and 32-lane transposing b64 reads of
// 4 consecutive k-rows (the NN W tile, 32 chunks per row).
__device__ __forceinline__ int swz_rows(int r) {
    return CPR == 8 ? (((r >> 1) & 7) ^ ((r & 1) << 2)) : ((r >> 2) & 3);
}
__device__ __forceinline__ int swz_w(int k) { return 4 * (k & 3); }

template <bool NN, int EPI, bool MULTI>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmParams P) {
    extern __shared__ uint4 gemm_smem[];
    char *smem = (char *)gemm_smem;
    const uint32_t smem_lds = (uint32_t)(uintptr_t)(lds_char *)smem;

    int tmi, tni;
    tile_coords(blockIdx.x, gridDim.x, P.tiles_m, P.tiles_n, tmi, tni);
    const int m0 = tmi * GBM, n0 = tni * GBN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, lhi = lane >> 5;

    f32x16_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    const size_t K2 = (size_t)P.K * 2, N2 = (size_t)P.N * 2;
    auto clamp_bytes = [](uint64_t v) { return (uint32_t)(v < 0x7FFFFFF0ull ? v : 0x7FFFFFF0ull); };
    const sgpr4_t dA = make_desc(P.Arow + (size_t)m0 * P.K, clamp_bytes((uint64_t)(P.M - m0) * K2));
    const sgpr4_t dBt = make_desc(P.Bcol + (size_t)n0 * P.K, NN ? 0u : clamp_bytes((uint64_t)(P.N - n0) * K2));
    const uint32_t nn_maxrows = 0x7FFFFFF0u / (uint32_t)N2;

    // ---- per-lane load geometry (constant over the K loop)
    // K-contiguous tiles: instruction j of this wave fills rows (wave*LPW+j)*RPI ..
    constexpr int RPI = 1024 / ROWB;  // rows per 1-KiB instruction
    uint32_t offK[LPW];   // byte offset of this lane's 16 B inside the global row panel (k0 = 0)
    int colK[LPW];        // its first column (for the K tail test)
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int r = (wave * LPW + j) * RPI + lane / CPR;
        const int c = (lane % CPR) ^ swz_rows(r);
        offK[j] = (uint32_t)(r * K2 + c * 16);
        colK[j] = c * 8;
    }
    // NN W tile: instruction j fills k-rows (wave*LPW+j)*2 .. +1, 32 chunks each
    uint32_t offW[LPW];
    if (NN) {
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int kr = (wave * LPW + j) * 2 + lane / 32;
            const int c = (lane % 32) ^ swz_w(kr);
            offW[j] = (uint32_t)(kr * N2 + (size_t)(n0 + c * 8) * 2);
        }
    }

    auto issue_loads = [&](int k0, int stage) {
        const uint32_t sa = smem_lds + stage * STAGE_BYTES + wave * LPW * 1024;
        const uint32_t sb = sa + TILE_BYTES;
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const uint32_t off = (k0 + colK[j] < P.K) ? offK[j] + (uint32_t)(k0 * 2) : kOOB;
            dma16(dA, off, sa + j * 1024);
        }
        if (NN) {
            const int kk = min(k0, P.K);
            const uint32_t rows = (uint32_t)min(P.K - kk, (int)nn_maxrows);
            const sgpr4_t dB = make_desc(P.Bcol + (size_t)kk * P.N, rows * (uint32_t)N2);
#pragma unroll
            for (int j = 0; j < LPW; ++j) dma16(dB, offW[j], sb + j * 1024);
        } else {
#pragma unroll
            for (int j = 0; j < LPW; ++j) {
                const uint32_t off = (k0 + colK[j] < P.K) ? offK[j] + (uint32_t)(k0 * 2) : kOOB;
                dma16(dBt, off, sb + j * 1024);
            }
        }
    };

    // ---- fragment reads
    int rowA[4], swA[4], rowB[4], swB[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        rowA[t] = wm * 128 + t * 32 + l32;
        swA[t] = swz_rows(rowA[t]);
        rowB[t] = wn * 128 + t * 32 + l32;
        swB[t] = swz_rows(rowB[t]);
    }
    // NN transposing reads: lane = 16*G + a; source row k = 8*(G>>1) + (a>>2) (+4),
    // chunk (col base)/8 + ((a&3)>>1), byte (a&1)*8 inside the chunk
    const int trG = lane >> 4, tra = lane & 15;
    const int tr_k = 8 * (trG >> 1) + (tra >> 2);
    const int tr_c = (wn * 128 + (trG & 1) * 16) / 8 + ((tra & 3) >> 1);
    const int tr_b = (tra & 1) * 8;

    uint4 af[2][4], bf[2][4];
    // One fragment (t-th of the row side if which == 0, of the column side if
    // which == 1) of sub-step ks from LDS stage `stage` into register slot `slot`.
    auto read_frag = [&](int stage, int ks, int slot, int which, int t) {
        const char *sa = smem + stage * STAGE_BYTES;
        const char *sb = sa + TILE_BYTES;
        const int c = 2 * ks + lhi;
        if (which == 0) {
            af[slot][t] = *(const uint4 *)(sa + rowA[t] * ROWB + ((c ^ swA[t]) << 4));
        } else if (NN) {
            const int k = ks * 16 + tr_k;
            const int ch = tr_c + 4 * t;
            const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s_t *)((lds_char *)sb + k * 512 + ((ch ^ swz_w(k)) << 4) + tr_b));
            const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s_t *)((lds_char *)sb + (k + 4) * 512 + ((ch ^ swz_w(k + 4)) << 4) + tr_b));
            const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
            bf[slot][t] = make_uint4(l2.x, l2.y, h2.x, h2.y);
        } else {
            bf[slot][t] = *(const uint4 *)(sb + rowB[t] * ROWB + ((c ^ swB[t]) << 4));
        }
    };
    auto read_frags = [&](int stage, int ks, int slot) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            read_frag(stage, ks, slot, 0, t);
            read_frag(stage, ks, slot, 1, t);
        }
    };

    // DMA of one operand tile slice: load j (0..2*LPW-1) of tile k0 into `stage`
    auto dma_one = [&](int k0, int stage, int j) {
        const uint32_t sa = smem_lds + stage * STAGE_BYTES + wave * LPW * 1024;
        if (j < LPW) {
            const uint32_t off = (k0 + colK[j] < P.K) ? offK[j] + (uint32_t)(k0 * 2) : kOOB;
            dma16(dA, off, sa + j * 1024);
        } else {
            const int jj = j - LPW;
            const uint32_t sb = sa + TILE_BYTES;
            if (NN) {
                const int kk = min(k0, P.K);
                const uint32_t rows = (uint32_t)min(P.K - kk, (int)nn_maxrows);
                const sgpr4_t dB = make_desc(P.Bcol + (size_t)kk * P.N, rows * (uint32_t)N2);
                dma16(dB, offW[jj], sb + jj * 1024);
            } else {
                const uint32_t off = (k0 + colK[jj] < P.K) ? offK[jj] + (uint32_t)(k0 * 2) : kOOB;
                dma16(dBt, off, sb + jj * 1024);
            }
        }
    };

    constexpr int KS = BK / 16;
    constexpr int NDMA = 2 * LPW;                 // DMA instructions per wave per tile
    constexpr int INFLIGHT = (NST - 2) * NDMA;    // loads allowed outstanding at a stage switch
    // 16 MFMAs of slot `sl`; MFMA i is followed by the i-th item of the side
    // work: fragment reads of (rstage, rks) into slot `rsl` for i < 8 and DMA
    // loads d0 + i/2 (every other MFMA) while they last.
    auto mfma_group = [&](int sl, bool do_read, int rstage, int rks, int rsl, int dk0, int dstage, int d0, int dn) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int tm = i >> 2, tn = i & 3;
            acc[tm][tn] = mfma32x32x16(bf[sl][tn], af[sl][tm], acc[tm][tn]);
            if (do_read && i < 8) read_frag(rstage, rks, rsl, i >> 2, i & 3);
            if ((i & 1) == 0 && (i >> 1) < dn) dma_one(dk0, dstage, d0 + (i >> 1));
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int nk = (P.K + BK - 1) / BK;
#pragma unroll
    for (int st = 0; st < NST - 1; ++st)
#pragma unroll
        for (int j = 0; j < NDMA; ++j) dma_one(st * BK, st, j);
    wait_vmcnt<INFLIGHT>();
    __syncthreads();
    read_frags(0, 0, 0);
    int stage = 0, lstage = NST - 1;
    for (int kt = 0; kt < nk; ++kt) {
        const int kload = (kt + NST - 1) * BK;
        // sub-steps 0..KS-2: MFMAs of ks with reads of ks+1; the tile's DMA
        // loads are spread over the first sub-steps (8 per sub-step)
#pragma unroll
        for (int ks = 0; ks < KS - 1; ++ks) {
            const int d0 = ks * 8;
            const int dn = d0 < NDMA ? min(8, NDMA - d0) : 0;
            mfma_group(ks & 1, true, stage, ks + 1, (ks + 1) & 1, kload, lstage, d0, dn);
        }
        if ((KS - 1) * 8 < NDMA) {
#pragma unroll
            for (int j = (KS - 1) * 8; j < NDMA; ++j) dma_one(kload, lstage, j);
        }
        wait_vmcnt<INFLIGHT>();
        __syncthreads();
        stage = stage + 1 == NST ? 0 : stage + 1;
        lstage = lstage + 1 == NST ? 0 : lstage + 1;
        // last sub-step after the barrier, overlapping the next tile's first reads
        mfma_group((KS - 1) & 1, kt + 1 < nk, stage, 0, 0, 0, 0, 0, 0);
    }
    wait_vmcnt<0>();

    const int wrow0 = m0 + wm * 128;  // first row of this wave
    const int wcol0 = n0 + wn * 128;  // first column of this wave

    // ---- F2: alpha * S * B accumulated into acc
    if (EPI == 1) {
        int s_begin = 0, s_end = 1;
        if (MULTI) {
            s_begin = first_segment(P, wrow0);
            s_end = P.nseg;
        }
        for (int s = s_begin; s < s_end; ++s) {
            if (MULTI && P.seg_off[s] >= (int64_t)(wrow0 + 128)) break;
            ExtItem it;
            if (!get_item<EPI, MULTI>(P, s, it)) continue;
            if (it.hi <= wrow0 || it.lo >= wrow0 + 128) continue;
            for (int rr0 = 0; rr0 < it.r; rr0 += 16) {
                uint4 cf[4];
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) cf[tn] = col_ext_frag<EPI>(P, it, wcol0 + tn * 32 + l32, rr0, lane);
#pragma unroll
                for (int tm = 0; tm < 4; ++tm) {
                    uint4 hi, lo;
                    row_ext_frags(P, it, wrow0 + tm * 32 + l32, rr0, lane, hi, lo);
#pragma unroll
                    for (int tn = 0; tn < 4; ++tn) {
                        acc[tm][tn] = mfma32x32x16(cf[tn], hi, acc[tm][tn]);
                        acc[tm][tn] = mfma32x32x16(cf[tn], lo, acc[tm][tn]);
                    }
                }
            }
        }
    }

    // ---- output (B3 adds the masked rank-deep term one 32-row band at a time)
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(P.C + (size_t)m0 * P.N, (size_t)(P.M - m0) * N2);
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        const int row = wrow0 + tm * 32 + l32;
        f32x16_t acc2[4];
        if (EPI == 2) {
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc2[tn][v] = 0.f;
            const int band0 = wrow0 + tm * 32;
            int s_begin = 0, s_end = 1;
            if (MULTI) {
                s_begin = first_segment(P, band0);
                s_end = P.nseg;
            }
            for (int s = s_begin; s < s_end; ++s) {
                if (MULTI && P.seg_off[s] >= (int64_t)(band0 + 32)) break;
                ExtItem it;
                if (!get_item<EPI, MULTI>(P, s, it)) continue;
                if (it.hi <= band0 || it.lo >= band0 + 32) continue;
                for (int rr0 = 0; rr0 < it.r; rr0 += 16) {
                    uint4 hi, lo;
                    row_ext_frags(P, it, row, rr0, lane, hi, lo);
#pragma unroll
                    for (int tn = 0; tn < 4; ++tn) {
                        const uint4 cf = col_ext_frag<EPI>(P, it, wcol0 + tn * 32 + l32, rr0, lane);
                        acc2[tn] = mfma32x32x16(cf, hi, acc2[tn]);
                        acc2[tn] = mfma32x32x16(cf, lo, acc2[tn]);
                    }
                }
            }
        }
        if (row < P.M) {
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) {
                const int tcol = wcol0 + tn * 32;
                if (tcol >= P.N) continue;
                uint32_t kw = 0xFFFFFFFFu;
                if (EPI == 2 && P.keep != nullptr) kw = P.keep[(size_t)row * P.KW + (tcol >> 5)];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int cofs = 8 * q + 4 * lhi;
                    const int col = tcol + cofs;
                    if (col >= P.N) continue;
                    uint32_t h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float v = acc[tm][tn][4 * q + e];
                        if (EPI == 2) {
                            if ((kw >> (cofs + e)) & 1u) v += acc2[tn][4 * q + e];
                        }
                        h[e] = f32_to_bf16_rne(v);
                    }
                    __builtin_amdgcn_raw_buffer_store_b64(
                        __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int,
                                           make_uint2(pack2(h[0], h[1]), pack2(h[2], h[3]))),
                        rC, (uint32_t)((size_t)(row - m0) * N2 + (size_t)col * 2), 0, 0);
                }
            }
        }
    }
}

size_t gemm_lds_bytes() { return (size_t)NST * STAGE_BYTES; }

template <bool NN, int EPI, bool MULTI>
static hipError_t launch_gemm_t(const GemmParams &P, hipStream_t stream, const char *name) {
    const size_t lds = gemm_lds_bytes();
    const int G = P.tiles_m * P.tiles_n;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm_kernel<NN, EPI, MULTI>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    (void)hipGetLastError();
    const int slot = prof_begin(name, stream);
    hipLaunchKernelGGL((gemm_kernel<NN, EPI, MULTI>), dim3(G), dim3(256), lds, stream, P);
    hipError_t e = hipGetLastError();
    prof_end(slot, stream);
    return e;
}

hipError_t launch_gemm(bool nn, int epi, const void *Arow, const void *Bcol, void *C, int M, int N,
                       int K, const float *Sx, int RS, const uint32_t *keep, int KW,
                       const AdapterSource &src, hipStream_t stream) {
    GemmParams P;
    P.Arow = (const uint16_t *)Arow;
    P.Bcol = (const uint16_t *)Bcol;
    P.C = (uint16_t *)C;
    P.M = M;
    P.N = N;
    P.K = K;
    P.tiles_m = (M + GBM - 1) / GBM;
    P.tiles_n = (N + GBN - 1) / GBN;
    P.Sx = Sx;
    P.RS = RS;
    P.keep = keep;
    P.KW = KW;
    P.ext = (const uint16_t *)(epi == 1 ? src.B : src.A);
    P.ext_r = src.r;
    P.ext_scale = epi == 1 ? src.alpha : drop_scale(src.p);
    P.adapters = src.table;
    P.num_adapters = src.num_adapters;
    P.r_cap = src.r_cap;
    P.seg_off = src.seg_off;
    P.seg_adapter = src.seg_adapter;
    P.nseg = src.num_segments;
    if (P.tiles_m == 0 || P.tiles_n == 0) return hipSuccess;
    const bool multi = src.table != nullptr;
    if (nn) {
        if (epi == 0) return launch_gemm_t<true, 0, false>(P, stream, "gemm_frozen_fwd");
        if (epi == 1) return multi ? launch_gemm_t<true, 1, true>(P, stream, "gemm_f2_fwd_lora")
                                   : launch_gemm_t<true, 1, false>(P, stream, "gemm_f2_fwd_lora");
    } else {
        if (epi == 0) return launch_gemm_t<false, 0, false>(P, stream, "gemm_frozen_bwd");
        if (epi == 2) return multi ? launch_gemm_t<false, 2, true>(P, stream, "gemm_b3_bwd_dx")
                                   : launch_gemm_t<false, 2, false>(P, stream, "gemm_b3_bwd_dx");
    }
    return hipErrorInvalidValue;
}

}  // namespace lora
