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

constexpr int GBM = 256, GBN = 256, GBK = 64, GLD = GBK + 8;

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

__device__ __forceinline__ uint4 ld16_or_zero(const uint16_t *p, bool ok) {
    return ok ? *(const uint4 *)p : make_uint4(0, 0, 0, 0);
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

template <bool NN, int EPI, bool MULTI>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmParams P) {
    extern __shared__ uint4 gemm_smem[];
    uint16_t *As = (uint16_t *)gemm_smem;  // [2][GBM][GLD]
    uint16_t *Bs = As + 2 * GBM * GLD;     // [2][GBN][GLD]

    int tmi, tni;
    tile_coords(blockIdx.x, gridDim.x, P.tiles_m, P.tiles_n, tmi, tni);
    const int m0 = tmi * GBM, n0 = tni * GBN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, lhi = lane >> 5;

    f32x16_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    // global -> register staging
    uint4 ra[8], rb[8];
    const int a_row = tid >> 3, a_col = (tid & 7) * 8;     // row-side / nt col-side
    const int nn_kb = tid & 7, nn_nb = tid >> 3;            // nn col-side 8x8 block

    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int row = m0 + c * 32 + a_row, col = k0 + a_col;
            ra[c] = ld16_or_zero(P.Arow + (size_t)row * P.K + col, row < P.M && col < P.K);
        }
        if (NN) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int krow = k0 + nn_kb * 8 + e, col = n0 + nn_nb * 8;
                rb[e] = ld16_or_zero(P.Bcol + (size_t)krow * P.N + col, krow < P.K && col < P.N);
            }
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int nrow = n0 + c * 32 + a_row, col = k0 + a_col;
                rb[c] = ld16_or_zero(P.Bcol + (size_t)nrow * P.K + col, nrow < P.N && col < P.K);
            }
        }
    };
    auto store_tiles = [&](int buf) {
        uint16_t *as = As + buf * GBM * GLD;
        uint16_t *bs = Bs + buf * GBN * GLD;
#pragma unroll
        for (int c = 0; c < 8; ++c) *(uint4 *)&as[(c * 32 + a_row) * GLD + a_col] = ra[c];
        if (NN) {
            uint4 o[8];
            transpose8x8(rb, o);
#pragma unroll
            for (int c = 0; c < 8; ++c) *(uint4 *)&bs[(nn_nb * 8 + c) * GLD + nn_kb * 8] = o[c];
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) *(uint4 *)&bs[(c * 32 + a_row) * GLD + a_col] = rb[c];
        }
    };

    const int nk = (P.K + GBK - 1) / GBK;
    if (nk > 0) {
        load_tiles(0);
        store_tiles(0);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_tiles((kt + 1) * GBK);
        const uint16_t *as = As + cur * GBM * GLD;
        const uint16_t *bs = Bs + cur * GBN * GLD;
#pragma unroll
        for (int ks = 0; ks < GBK / 16; ++ks) {
            uint4 af[4], bf[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                af[t] = *(const uint4 *)&as[(wm * 128 + t * 32 + l32) * GLD + ks * 16 + lhi * 8];
                bf[t] = *(const uint4 *)&bs[(wn * 128 + t * 32 + l32) * GLD + ks * 16 + lhi * 8];
            }
#pragma unroll
            for (int tm = 0; tm < 4; ++tm)
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = mfma32x32x16(bf[tn], af[tm], acc[tm][tn]);
        }
        if (kt + 1 < nk) store_tiles(cur ^ 1);
        __syncthreads();
    }

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
                    *(uint2 *)(P.C + (size_t)row * P.N + col) = make_uint2(pack2(h[0], h[1]), pack2(h[2], h[3]));
                }
            }
        }
    }
}

size_t gemm_lds_bytes() { return (size_t)2 * (GBM + GBN) * GLD * sizeof(uint16_t); }

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
