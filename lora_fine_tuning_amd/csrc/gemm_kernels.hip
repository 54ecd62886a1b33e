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
// Tiling: a 256 x 256 output tile per work-group of 4 waves (2 x 2, one wave
// per SIMD), each wave an 8 x 8 grid of v_mfma_f32_16x16x32_bf16 tiles with
// fp32 accumulators.  (The 16x16x32 form moves a quarter of the accumulator
// bytes per flop of the 32x32x16 form; under sustained load the chip holds a
// clock about 15% higher with it.)  The column-side operand is the MFMA's
// first source, so each lane ends with 4 consecutive output columns of one
// row (8-byte stores).
//
// K advances in 64-deep stages through a 2-stage LDS ring (2 x 64 KiB) filled
// by direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds); a stage is two
// 32-deep MFMA steps.  The loads of stage t+2 are issued right after the
// barrier that retires stage t's buffer, interleaved with the MFMAs of the
// second step of stage t and so covered by two MFMA steps.  Fragment reads for
// the next step interleave with the MFMAs of the current one (double-buffered
// fragments).  K-contiguous tiles use 128-byte rows with a 16-byte-chunk XOR
// swizzle (conflict-free 16-lane b128 reads of 16 consecutive rows); the
// forward's W tile is k-row major (512-byte rows, n contiguous) and is read
// with ds_read_b64_tr_b16, which gives each lane 4 consecutive k of one
// column; its swizzle keeps the 32 lanes of a half-wave (8 k-rows x 32 bytes)
// on distinct banks.  Work-group ids are remapped so each XCD gets a
// contiguous range of tiles, visited in groups of 8 row panels.
//
// The LoRA terms run after the K loop as extra rank-deep MFMA steps whose
// operands come straight from global memory: fp32 S (or dS) as hi+lo bf16
// pairs times B (or A).  For the masked backward term the rank-deep product
// goes to a second accumulator, one 16-row band at a time, and is added under
// the stored keep bits.  Mixed-adapter tiles run one such pass per segment
// overlapping the tile (rows of other segments contribute zero).
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace lora {

constexpr int GBM = 256, GBN = 256;
constexpr int kStoreNT = 2;  // buffer-store cache policy: nt (non-temporal)

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
    // multi adapter: S / dS rows and mask rows meet the fast epilogue's
    // alignment (RS % 8 == 0, 16-byte aligned; KW % 4 == 0, 16-byte aligned)
    int multi_fast;
    // mask rows 16-byte aligned with KW % 4 == 0 (one 16-byte load per row)
    int keep16;
    // epi 3 (forward, ranks 33..128): the LoRA term as kx = 2*RP extra K
    // columns -- S2 (M x kx bf16: alpha*S split, [hi | lo] of RP ranks each)
    // against B's rows (rank j for extra column j and RP + j; past r zero)
    const uint16_t *S2;
    int kx;
    // FAST == 3 (forward at p = 0, [W | A] as one operand): A (K x ext_r) and
    // the S output (M x ext_r fp32, written by the tiles of column 0)
    const uint16_t *catA;
    float *Sout;
    // B3 with A staged in LDS: optional rows of [hi | lo] bf16 of s*dS (the
    // row's adapter's rpa ranks each, dss_ld apart), read instead of dS
    const uint16_t *dss;
    int dss_ld;
};

// acc += a * b with the accumulator in VGPRs (the AGPRs hold the product's
// tiles); like the in-place form, its latency is not modelled, so its result
// is read only after mfma_drain().
__device__ __forceinline__ void mfma16x16x32_vacc(f32x4_t &acc, const uint4 &a, const uint4 &b) {
    typedef int i32x4_t __attribute__((ext_vector_type(4)));
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                 : "+v"(acc)
                 : "v"(__builtin_bit_cast(i32x4_t, a)), "v"(__builtin_bit_cast(i32x4_t, b)));
}
// acc = a * b (the accumulator input is the constant 0, so no VALU write of
// it can be in flight when the MFMA reads it)
__device__ __forceinline__ void mfma16x16x32_vfirst(f32x4_t &acc, const uint4 &a, const uint4 &b) {
    typedef int i32x4_t __attribute__((ext_vector_type(4)));
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0"
                 : "=v"(acc)
                 : "v"(__builtin_bit_cast(i32x4_t, a)), "v"(__builtin_bit_cast(i32x4_t, b)));
}

// m ? b : a bit by bit (m is 0 or ~0, wave-uniform).  Written as one
// v_bfi_b32 so the compiler cannot turn a select of two fragment registers
// into an indexed access of the fragment array (which would put it in
// scratch memory).
__device__ __forceinline__ uint32_t bitsel(uint32_t m, uint32_t b, uint32_t a) {
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(m), "v"(b), "v"(a));
    return r;
}

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

// Rank-deep MFMA step, row side: row_ext_load reads fp32 S/dS of `row` for
// ranks rr0 + 8*(lane/16) .. +7; rows outside [lo, hi) and ranks past r read
// as zero (out-of-range buffer offsets, no branches).  rS starts at row `row0`
// (the wave's first row), so offsets stay small.  `vec`: r and RS are
// multiples of 8 and Sx is 16-byte aligned, so the 8 values are two aligned
// 16-byte loads.  row_ext_split multiplies them by the item's scale and splits
// them into hi/lo fragments; row_ext_frags does both.
__device__ __forceinline__ void row_ext_load(const GemmParams &P, __amdgpu_buffer_rsrc_t rS, int row0,
                                             const ExtItem &it, int row, int rr0, int lane, bool vec,
                                             float (&v)[8]) {
    const bool ok = row >= it.lo && row < it.hi;
    const int rb = rr0 + 8 * (lane >> 4);
    const uint32_t base = (uint32_t)((row - row0) * P.RS + rb) * 4u;
    if (vec) {
        const uint32_t off = (ok && rb < it.r) ? base : kOOB;
        const float4 a = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rS, off, 0, 0));
        const float4 b = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rS, off == kOOB ? kOOB : off + 16, 0, 0));
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t off = (ok && rb + e < it.r) ? base + 4u * e : kOOB;
            v[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS, off, 0, 0));
        }
    }
}

// The loaded values times the item's scale, as hi / lo bf16 fragments.
__device__ __forceinline__ void row_ext_split(const ExtItem &it, const float (&v)[8], uint4 &hi, uint4 &lo) {
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = v[e] * it.scale;
    split_frag(w, hi, lo);
}

__device__ __forceinline__ void row_ext_frags(const GemmParams &P, __amdgpu_buffer_rsrc_t rS, int row0,
                                              const ExtItem &it, int row, int rr0, int lane, bool vec,
                                              uint4 &hi, uint4 &lo) {
    float v[8];
    row_ext_load(P, rS, row0, it, row, rr0, lane, vec, v);
    row_ext_split(it, v, hi, lo);
}

// Rank-deep step, column side: 8 consecutive ranks of output column `col`
// (zero past r or N).  epi 1 reads B[rr][col] (stride N); epi 2 reads
// A[col][rr], 16 contiguous bytes, one load when `vec` (r a multiple of 8, A
// 16-byte aligned).  rW is a buffer resource over B (r x N) or A (N x r)
// starting at column `col0` (B's whole rows stay under 2 GiB: checked by the
// launcher).
template <int EPI>
__device__ __forceinline__ uint4 col_ext_frag(const GemmParams &P, __amdgpu_buffer_rsrc_t rW, int col0,
                                              const ExtItem &it, int col, int rr0, int lane, bool vec) {
    const bool cok = col < P.N;
    const int rb = rr0 + 8 * (lane >> 4);
    const int cr = col - col0;
    if (EPI == 2 && vec) {
        const uint32_t off = (cok && rb < it.r) ? (uint32_t)(cr * it.r + rb) * 2u : kOOB;
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rW, off, 0, 0));
    }
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int rr = rb + e;
        const uint32_t idx = EPI == 1 ? (uint32_t)rr * (uint32_t)P.N + (uint32_t)cr : (uint32_t)(cr * it.r + rr);
        const uint32_t off = (cok && rr < it.r) ? idx * 2u : kOOB;
        h[e] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rW, off, 0, 0);
    }
    return make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
}

// Buffer resource over an adapter's rank-side matrix (r x N for B, N x r for
// A) from column col0 on.
template <int EPI>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ext_rsrc(const GemmParams &P, const ExtItem &it, int col0) {
    const uint64_t total = (uint64_t)it.r * (uint64_t)P.N * 2u;
    const uint64_t skip = (uint64_t)min(col0, P.N) * (EPI == 1 ? 2u : 2u * (uint64_t)it.r);
    return make_rsrc(it.w + (EPI == 1 ? (size_t)min(col0, P.N) : (size_t)min(col0, P.N) * it.r), total - skip);
}

// Every field of an item as a wave-uniform value (SGPRs).
__device__ __forceinline__ ExtItem uniform_item(const ExtItem &it) {
    ExtItem u;
    u.lo = __builtin_amdgcn_readfirstlane(it.lo);
    u.hi = __builtin_amdgcn_readfirstlane(it.hi);
    u.r = __builtin_amdgcn_readfirstlane(it.r);
    u.scale = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, it.scale)));
    const uint64_t w = (uint64_t)(uintptr_t)it.w;
    const uint32_t wl = __builtin_amdgcn_readfirstlane((uint32_t)w), wh = __builtin_amdgcn_readfirstlane((uint32_t)(w >> 32));
    u.w = (const uint16_t *)(uintptr_t)(((uint64_t)wh << 32) | wl);
    return u;
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
    // s is the same in every lane at every call, so the item is too; saying
    // so keeps its fields in SGPRs (a buffer resource built from VGPR fields
    // turns each load through it into a loop over the distinct values)
    it = uniform_item(it);
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


// ---- B3 with the rank-side matrix staged in LDS.  The adapter items of one
// 256-row tile (at most two; consecutive segments of one adapter count as
// one), each with r <= 128, r a multiple of 8 and a 16-byte aligned A.  Every
// thread of the work-group computes the same plan.
struct TileItems {
    int n;
    ExtItem it[2];  // indexed by constants only (no dynamic index: registers, not scratch)
    int rp[2];      // ranks rounded up to a multiple of 32
};


template <bool MULTI>
__device__ __forceinline__ bool plan_tile_items(const GemmParams &P, int m0, TileItems &ti) {
    const int rend = min(m0 + GBM, P.M);
    int n = 0;
    ExtItem a{}, b{};
    if (!MULTI) {
        get_item<2, false>(P, 0, a);
        n = 1;
    } else {
        for (int s = first_segment(P, m0); s < P.nseg && P.seg_off[s] < (int64_t)rend; ++s) {
            ExtItem it;
            if (!get_item<2, true>(P, s, it)) continue;
            if (it.hi <= m0 || it.lo >= rend) continue;
            if (n == 1 && it.w == a.w && it.r == a.r && it.scale == a.scale && it.lo == a.hi) {
                a.hi = it.hi;  // the same adapter goes on: one item
                continue;
            }
            if (n == 2) return false;
            if (n == 0) a = it;
            else b = it;
            ++n;
        }
        if (n == 0) return false;
    }
    if (a.r > 128 || (a.r & 7) != 0 || (((uintptr_t)a.w) & 15) != 0) return false;
    if (n == 2 && (b.r > 128 || (b.r & 7) != 0 || (((uintptr_t)b.w) & 15) != 0)) return false;
    ti.n = __builtin_amdgcn_readfirstlane(n);
    ti.it[0] = uniform_item(a);
    ti.it[1] = uniform_item(b);
    ti.rp[0] = (ti.it[0].r + 31) & ~31;
    ti.rp[1] = (ti.it[1].r + 31) & ~31;
    return true;
}

// LDS slab of 64 ranks of A for the tile's 256 columns: 128-byte column rows,
// the 16-byte chunk holding ranks 8q .. 8q+7 of column c at chunk position
// q ^ ((c >> 1) & 7) (16 consecutive columns read at one rank chunk hit 16
// distinct 16-byte bank groups).
__device__ __forceinline__ uint32_t slab_off(int c, int q) { return (uint32_t)(c * 128 + ((q ^ ((c >> 1) & 7)) << 4)); }

constexpr int BK = 64;              // K depth of one LDS stage
constexpr int NST = 2;              // stages in the LDS ring
constexpr int ROWB = BK * 2;        // bytes per LDS row of a K-contiguous tile
constexpr int CPR = BK / 8;         // 16-byte chunks per such row
constexpr int TILE_BYTES = GBM * ROWB;  // one operand tile (the NN W tile is BK x 512 B, same size)
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr int LPW = BK / 8;         // 1-KiB direct-to-LDS loads per wave per operand per stage
constexpr int NDMA = 2 * LPW;       // DMA instructions per wave per stage
constexpr int NT16 = 8;             // 16 x 16 MFMA tiles per wave side

// XOR swizzle of the 16-byte chunks of a 128-byte row: 16 consecutive rows
// read at one chunk position land on 16 distinct chunks of a 256-byte bank window.
__device__ __forceinline__ int swz_rows(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }
// W tile (512-byte k-rows): k-rows {0..3, 8..11} (mod 16) get 8 distinct even
// chunk offsets, so the 8 rows x 32 bytes of a half-wave transposing read are
// conflict-free.
__device__ __forceinline__ int swz_w(int k) { return (4 * (k & 3)) ^ (2 * ((k >> 3) & 1)); }

// FAST != 0 (single adapter, r <= 32 and a multiple of 8, 16-byte aligned S /
// dS, rank-side matrix and mask rows; chosen by the host): the epilogue issues
// all its loads up front.  FAST == 2 is the r <= 16 form that folds the two
// halves of the split row side into one MFMA.  Each is its own instantiation
// so no kernel merges two epilogues.
//
// FAST == 3 (forward only, p = 0, r 8 or 16): the concatenated form of the
// FALQON notes (section 5.2, W' = [W; A] as one operand).  Each tile forms
// its own 256 x 16 block of S = X A inside the K loop -- A's 64 x 16 slice
// rides along with every stage and each wave forms S for 64 of the tile's
// rows from the row fragments it already holds (about 6% more MFMA work than
// the 256 x 256 product) -- and then applies alpha S B in the FAST == 2
// epilogue from LDS.  No separate pass over X forms S; the tiles of column 0 also
// write S out for the backward.
template <bool NN, int EPI, bool MULTI, int FAST>
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
    const int l16 = lane & 15, lg = lane >> 4;

    f32x4_t acc[NT16][NT16];
#pragma unroll
    for (int a = 0; a < NT16; ++a)
#pragma unroll
        for (int b = 0; b < NT16; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

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

    // epi 3: geometry of the extra K stages (S2 rows stride kx; B rows by
    // extra column, the W tile's chunk swizzle)
    constexpr bool KEXT = EPI == 3;
    const int nkx = (P.K + BK - 1) / BK;  // stages of X / W before the extra ones
    uint32_t offX2[LPW];
    if (KEXT) {
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int r = (wave * LPW + j) * RPI + lane / CPR;
            const int c = (lane % CPR) ^ swz_rows(r);
            offX2[j] = (uint32_t)(r * P.kx * 2 + c * 16);
        }
    }
    const sgpr4_t dX2 = make_desc(KEXT ? P.S2 + (size_t)m0 * P.kx : P.Arow,
                                  KEXT ? clamp_bytes((uint64_t)(P.M - m0) * P.kx * 2u) : 0u);
    const sgpr4_t dBx = make_desc(P.ext, KEXT ? clamp_bytes((uint64_t)P.ext_r * N2) : 0u);

    // DMA load j (0..NDMA-1) of the stage starting at k0 into LDS stage
    // `stage`; extra_c (compile-time) selects an extra-K stage of epi 3
    auto dma_one = [&](int k0, int stage, int j, auto extra_c) {
        constexpr bool EXTRA = decltype(extra_c)::value;
        const uint32_t sa = smem_lds + stage * STAGE_BYTES + wave * LPW * 1024;
        if constexpr (EXTRA) {
            const int kx0 = k0 - nkx * BK;  // first extra column of the stage
            if (j < LPW) {
                const uint32_t off = (kx0 + colK[j] < P.kx) ? offX2[j] + (uint32_t)(kx0 * 2) : kOOB;
                dma16(dX2, off, sa + j * 1024);
            } else {
                const int jj = j - LPW;
                const int kr = (wave * LPW + jj) * 2 + lane / 32;
                const int c = (lane % 32) ^ swz_w(kr);
                const int kp = kx0 + kr, rp = P.kx >> 1;
                const int brow = kp < rp ? kp : kp - rp;
                const uint32_t off = (kp < P.kx && brow < P.ext_r)
                    ? (uint32_t)(brow * N2 + (size_t)(n0 + c * 8) * 2) : kOOB;
                dma16(dBx, off, sa + TILE_BYTES + jj * 1024);
            }
            return;
        }
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

    // ---- fragment reads.  Row side: 16 rows x 32 K per tile, lane l reads row
    // l%16 of the tile, K chunk 4*ks + l/16; swz_rows of the row depends only
    // on l%16, so tile t is at a fixed 2048-byte stride.  Column side (nt): the
    // same on the B tile.
    const int swl = swz_rows(l16);
    int rdA[2], rdB[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        rdA[ks] = (wm * 128 + l16) * ROWB + (((4 * ks + lg) ^ swl) << 4);
        rdB[ks] = TILE_BYTES + (wn * 128 + l16) * ROWB + (((4 * ks + lg) ^ swl) << 4);
    }
    // NN transposing reads: within 16-lane group g (K slots 8g..8g+7) source
    // lane s points at k-row 8g + s/4 (+4 for the second read), columns
    // colbase + 4*(s%4) .. +3, so output lane s gets column colbase + s.  The
    // swizzle of those k-rows depends only on the lane, so each tile t has one
    // address; +4 rows is +2048 bytes and the second K step +16384.
    int rdW[NT16];
    if (NN) {
        const int tr_k = 8 * lg + (l16 >> 2);
        const int sww = swz_w(tr_k);
#pragma unroll
        for (int t = 0; t < NT16; ++t) {
            const int ch = (wn * 128 + t * 16) / 8 + ((l16 & 3) >> 1);
            rdW[t] = TILE_BYTES + tr_k * 512 + ((ch ^ sww) << 4) + (l16 & 1) * 8;
        }
    }

    uint4 af[2][NT16], bf[2][NT16];
    constexpr bool CAT = FAST == 3 && EPI == 1 && !MULTI;
    // FAST == 3: A's rows k0 .. k0+63 of a stage at 24 KiB past the ring +
    // 4 KiB per stage, 32 bytes (16 ranks; past r zero) per k-row; waves 0
    // and 1 load them, waves 2 and 3 load zeros into the stage's spare half
    // (every wave issues the same number of loads per stage)
    uint4 aAf[2], xsel = make_uint4(0u, 0u, 0u, 0u);
    const uint32_t wn_mask = wn ? ~0u : 0u;  // wave-uniform
    f32x4_t sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) sacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const sgpr4_t dAcat = make_desc(CAT ? (const void *)P.catA : (const void *)P.Arow,
                                    CAT ? clamp_bytes((uint64_t)P.K * (uint64_t)P.ext_r * 2u) : 0u);
    auto dma_a = [&](int k0, int stage) {
        const int kr = 32 * wave + (lane >> 1), ch = lane & 1;
        const uint32_t off = (wave < 2 && k0 + kr < P.K && 8 * ch < P.ext_r)
            ? ((uint32_t)(k0 + kr) * (uint32_t)P.ext_r + 8u * ch) * 2u : kOOB;
        dma16(dAcat, off, smem_lds + NST * STAGE_BYTES + 24576 + stage * 4096 + wave * 1024);
    };
    // column-side fragment of A for 32-deep step ks of a stage: lane l gets
    // rank l % 16 at K slots 8 (l / 16) .. +7 (two transposing reads of 4 k-rows)
    auto read_afrag = [&](int stage, int ks, int slot) {
        const lds_char *pa = (const lds_char *)smem + NST * STAGE_BYTES + 24576 + stage * 4096 +
                             (32 * ks + 8 * lg + (l16 >> 2)) * 32 + (l16 & 3) * 8;
        const uint2 lo = lds_read_tr4(pa), hi = lds_read_tr4(pa + 128);
        aAf[slot] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    };
    // the `which`-side fragment t of step ks (0/1) of LDS stage `stage` into slot `slot`
    auto read_frag = [&](int stage, int ks, int slot, int which, int t) {
        const char *base = smem + stage * STAGE_BYTES;
        if (which == 0) {
            af[slot][t] = *(const uint4 *)(base + rdA[ks] + t * 2048);
        } else if (NN) {
            const lds_char *p = (const lds_char *)base + rdW[t] + ks * 16384;
            const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t *)p);
            const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t *)(p + 2048));
            const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
            bf[slot][t] = make_uint4(l2.x, l2.y, h2.x, h2.y);
        } else {
            bf[slot][t] = *(const uint4 *)(base + rdB[ks] + t * 2048);
        }
    };

    // 64 MFMAs of fragment slot `sl`; MFMA i is followed by side work: for
    // i % 4 == 0 the fragment read i/4 of (rstage, rks) into slot rsl, and for
    // i % 4 == 2 the DMA load i/4 of the stage at dk0 into dstage.  READ, DMA
    // and EXTRA (the DMA is of an extra-K stage) are compile-time flags so the
    // MFMA stream carries no branches.
    auto mfma_step = [&](int sl, auto read_c, int rstage, int rks, int rsl, auto dma_c, int dk0, int dstage,
                         auto extra_c) __attribute__((always_inline)) {
        constexpr bool READ = decltype(read_c)::value, DMA = decltype(dma_c)::value;
#pragma unroll
        for (int i = 0; i < NT16 * NT16; ++i) {
            const int tm = i >> 3, tn = i & 7;
            mfma16x16x32_inplace(acc[tm][tn], bf[sl][tn], af[sl][tm]);
            if constexpr (READ) {
                if ((i & 3) == 0) read_frag(rstage, rks, rsl, (i >> 2) & 1, i >> 3);
            }
            if constexpr (DMA) {
                if ((i & 3) == 2) dma_one(dk0, dstage, i >> 2, extra_c);
            }
            if constexpr (CAT) {
                if constexpr (READ) {
                    if (i == 1) read_afrag(rstage, rks, rsl);
                }
                if constexpr (DMA) {
                    if (i == 63) dma_a(dk0, dstage);
                }
                // S of the wave's quarter of the tile's rows (row tiles 4 wn ..
                // 4 wn + 3 of its half), one MFMA after every 16 of the
                // product.  The row fragment is picked by select, not by a
                // branch, so the MFMA stream stays one basic block, 12 MFMAs
                // before the MFMA that reads it (far past the VALU-to-MFMA
                // operand hazard); the accumulators stay in VGPRs.
                if ((i & 15) == 3) {
                    const int t = i >> 4;
                    xsel.x = bitsel(wn_mask, af[sl][4 + t].x, af[sl][t].x);
                    xsel.y = bitsel(wn_mask, af[sl][4 + t].y, af[sl][t].y);
                    xsel.z = bitsel(wn_mask, af[sl][4 + t].z, af[sl][t].z);
                    xsel.w = bitsel(wn_mask, af[sl][4 + t].w, af[sl][t].w);
                }
                if ((i & 15) == 15) mfma16x16x32_vacc(sacc[i >> 4], aAf[sl], xsel);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;

    // ---- FAST == 2: the epilogue's operands go to the 32 KiB past the stage
    // ring by direct-to-LDS loads issued right after the prologue, so they
    // arrive during the K loop (whose first full wait covers them).  Layout
    // (byte offsets from the region's start):
    //   0      S / dS rows m0 .. m0+255, 64 bytes each (ranks 0..15; ranks at
    //          or past RS zero), 16-byte chunk c of row q at c ^ ((q >> 2) & 3)
    //   16384  F2: B ranks 0..15 x columns n0 .. n0+255, 512-byte rows with
    //          the W tile's chunk swizzle; B3: A rows n0 .. n0+255 (r bf16
    //          each) as one contiguous block
    //   24576  B3: mask words n0/32 .. +7 of rows m0 .. m0+255, 32 bytes each
    constexpr bool PF = (FAST == 2 || CAT) && EPI != 0 && !MULTI;
    constexpr int NPF = EPI == 2 ? 8 : CAT ? 2 : 6;  // prefetch loads per wave
    const uint32_t pf_lds = smem_lds + NST * STAGE_BYTES;
    auto epi_prefetch = [&]() {
        if (!CAT) {
            const sgpr4_t d = make_desc(P.Sx + (size_t)m0 * P.RS, clamp_bytes((uint64_t)(P.M - m0) * P.RS * 4u));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = 4 * wave + q, row = 16 * j + (lane >> 2);
                const int lc = (lane & 3) ^ ((row >> 2) & 3);
                const uint32_t off = (m0 + row < P.M && 4 * lc < P.RS) ? (uint32_t)(row * P.RS + 4 * lc) * 4u : kOOB;
                dma16(d, off, pf_lds + j * 1024);
            }
        }
        if (EPI == 1) {
            const sgpr4_t d = make_desc(P.ext, (uint32_t)P.ext_r * (uint32_t)N2);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int j = 2 * wave + q, kr = 2 * j + (lane >> 5);
                const int col = n0 + 8 * ((lane & 31) ^ swz_w(kr));
                const uint32_t off = (kr < P.ext_r && col < P.N) ? (uint32_t)(kr * P.N + col) * 2u : kOOB;
                dma16(d, off, pf_lds + 16384 + j * 1024);
            }
        } else {
            const uint32_t abytes = (uint32_t)P.N * (uint32_t)P.ext_r * 2u;
            const uint32_t a0 = (uint32_t)n0 * (uint32_t)P.ext_r * 2u, ablk = 256u * (uint32_t)P.ext_r * 2u;
            const sgpr4_t d = make_desc(P.ext, abytes);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int j = 2 * wave + q;
                const uint32_t b = (uint32_t)(j * 64 + lane) * 16u;
                dma16(d, (b < ablk && a0 + b < abytes) ? a0 + b : kOOB, pf_lds + 16384 + j * 1024);
            }
            const bool has_keep = P.keep != nullptr;
            const sgpr4_t dk = make_desc(has_keep ? P.keep + (size_t)m0 * P.KW : P.keep,
                                         has_keep ? clamp_bytes((uint64_t)(P.M - m0) * P.KW * 4u) : 0u);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int j = 2 * wave + q, row = 32 * j + (lane >> 1);
                const int w = (n0 >> 5) + 4 * (lane & 1);
                const uint32_t off = (has_keep && m0 + row < P.M && w < P.KW) ? (uint32_t)(row * P.KW + w) * 4u : kOOB;
                dma16(dk, off, pf_lds + 24576 + j * 1024);
            }
        }
    };

    const int nk = nkx + (KEXT ? (P.kx + BK - 1) / BK : 0);
    // prologue: stages 0 and 1 in flight, wait for stage 0
    if (KEXT && nkx < 1) {
#pragma unroll
        for (int j = 0; j < NDMA; ++j) dma_one(0, 0, j, std::true_type{});
    } else {
#pragma unroll
        for (int j = 0; j < NDMA; ++j) dma_one(0, 0, j, std::false_type{});
    }
    if constexpr (CAT) dma_a(0, 0);
    if (KEXT && nkx < 2) {
#pragma unroll
        for (int j = 0; j < NDMA; ++j) dma_one(BK, 1, j, std::true_type{});
    } else {
#pragma unroll
        for (int j = 0; j < NDMA; ++j) dma_one(BK, 1, j, std::false_type{});
    }
    if constexpr (CAT) dma_a(BK, 1);
    // B3 (not the all-loads-first forms): when the tile's items fit (see
    // plan_tile_items), A is staged in LDS for the epilogue.  The slab of the
    // first item's ranks 0..63 goes to the 32 KiB past the ring now, loaded
    // during the K loop; the rest follows the K loop into the idle ring.
    TileItems ti;
    bool lds_epi = false;
    auto slab_dma = [&](const ExtItem &it, int rbase, uint32_t dst) {
        // the item is the same in every lane: its address and size go to SGPRs
        const uint64_t ab = (uint64_t)P.N * (uint64_t)it.r * 2u;
        const uint64_t wp = (uint64_t)(uintptr_t)it.w;
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)wp);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(wp >> 32));
        const uint32_t nb = __builtin_amdgcn_readfirstlane((uint32_t)(ab < 0x7FFFFFF0ull ? ab : 0x7FFFFFF0ull));
        const sgpr4_t d = make_desc((const void *)(uintptr_t)(((uint64_t)hi << 32) | lo), nb);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int j = 8 * wave + q, c = 8 * j + (lane >> 3);
            const int lq = (lane & 7) ^ ((c >> 1) & 7);  // logical 8-rank chunk of the lane's 16 bytes
            const uint32_t off = (n0 + c < P.N && rbase + 8 * lq < it.r)
                ? ((uint32_t)(n0 + c) * (uint32_t)it.r + (uint32_t)(rbase + 8 * lq)) * 2u : kOOB;
            dma16(d, off, dst + j * 1024);
        }
    };
    if constexpr (EPI == 2 && FAST == 0) {
        const bool svec0 = (P.RS & 7) == 0 && (((uintptr_t)P.Sx) & 15) == 0;
        lds_epi = svec0 && (P.keep == nullptr || P.keep16) && plan_tile_items<MULTI>(P, m0, ti);
        // one item of rank <= 32 in a mixed batch: the all-loads-first epilogue below
        if (MULTI && lds_epi && ti.n == 1 && ti.it[0].r <= 32 && P.multi_fast) lds_epi = false;
        if (lds_epi) slab_dma(ti.it[0], 0, pf_lds);
    }
    if constexpr (PF) epi_prefetch();
    if (lds_epi) wait_vmcnt<NDMA + 8>();
    else wait_vmcnt<PF ? NDMA + NPF + (CAT ? 1 : 0) : NDMA>();
    asm volatile("" ::: "memory");  // keep the LDS reads below the barrier
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t < NT16; ++t) {
        read_frag(0, 0, 0, 0, t);
        read_frag(0, 0, 0, 1, t);
    }
    if constexpr (CAT) read_afrag(0, 0, 0);
    // No scalar load may still be in flight when the K loop starts (the
    // compiler sinks the epilogue's kernel-argument loads to here): one would
    // make it wait for every LDS read (lgkmcnt 0) at the top of each MFMA step
    // instead of only for the fragments the next MFMAs use.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
    // One stage: step 0 (reads of its step 1), then -- once stage kt+1 has
    // landed everywhere and stage kt's buffer is no longer read -- step 1 with
    // the reads of step 0 of stage kt+1 and the loads of stage kt+2 into the
    // buffer stage kt released.  The last two stages drop the loads / reads.
    auto stage_body = [&](int kt, auto read_next, auto load_next2, auto extra_c) __attribute__((always_inline)) {
        const int stage = kt & 1;
        mfma_step(0, T_{}, stage, 1, 1, F_{}, 0, 0, F_{});
        wait_vmcnt<0>();
        __syncthreads();
        mfma_step(1, read_next, stage ^ 1, 0, 0, load_next2, (kt + 2) * BK, stage, extra_c);
    };
    int kt = 0;
    // epi 3: stages whose loads (two ahead) are extra-K ones take their own
    // unrolled copy of the stage
    for (; kt + 2 < (KEXT ? min(nk, nkx) : nk); ++kt) stage_body(kt, T_{}, T_{}, F_{});
    if constexpr (KEXT) {
        for (; kt + 2 < nk; ++kt) stage_body(kt, T_{}, T_{}, T_{});
    }
    if (kt + 1 < nk) stage_body(kt++, T_{}, F_{}, F_{});
    if (kt < nk) stage_body(kt, F_{}, F_{}, F_{});
    mfma_drain();
    wait_vmcnt<0>();
    if constexpr (CAT) {
        // each wave's 64 rows of S go to the epilogue's S rows (fp32, 64
        // bytes per row, chunk c of row q at c ^ ((q >> 2) & 3)); the tiles
        // of column 0 also write them out
        lds_char *sp = (lds_char *)smem + NST * STAGE_BYTES;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int q = wm * 128 + wn * 64 + 16 * t + l16;
            *(f32x4_t *)(sp + q * 64 + ((lg ^ ((q >> 2) & 3)) << 4)) = sacc[t];
            if (tni == 0 && m0 + q < P.M && 4 * lg < P.ext_r)
                *(f32x4_t *)(P.Sout + (size_t)(m0 + q) * P.ext_r + 4 * lg) = sacc[t];
        }
    }

    const int wrow0 = m0 + wm * 128;  // first row of this wave
    const int wcol0 = n0 + wn * 128;  // first column of this wave

    const __amdgpu_buffer_rsrc_t rS = make_rsrc(P.Sx + (size_t)min(wrow0, P.M) * P.RS,
                                                (uint64_t)max(P.M - wrow0, 0) * (uint64_t)P.RS * 4u);
    const bool svec = (P.RS & 7) == 0 && (((uintptr_t)P.Sx) & 15) == 0;
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(P.C + (size_t)m0 * P.N, (size_t)(P.M - m0) * N2);

    // ---- output staging.  Each lane holds 4 consecutive columns of a row per
    // 16 x 16 tile, so direct stores would write 32-byte pieces of 16 rows
    // per instruction.  Instead the wave's 128 x 128 bf16 block goes to its
    // 32 KiB of the (now idle) stage ring -- every wave passed the K loop's
    // last barrier after its last ring read -- with the 16-byte chunks of each
    // 256-byte row XOR-swizzled by the row, and is written out as 1 KiB
    // stores of 4 whole rows (full cache lines).
    lds_char *cw = (lds_char *)smem + wave * 32768;
    auto c_put = [&](int tm, int tn, float x0, float x1, float x2, float x3) {
        const int r = tm * 16 + l16;
        const int ch = (2 * tn + (lg >> 1)) ^ (r & 15);
        *(uint2 *)(cw + r * 256 + ch * 16 + (lg & 1) * 8) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
    };
    auto c_flush = [&]() {
        const int cc = lane & 15;
        const int col = wcol0 + cc * 8;
#pragma unroll 4
        for (int it = 0; it < 32; ++it) {
            const int r = it * 4 + (lane >> 4);
            const uint4 v = *(const uint4 *)(cw + r * 256 + ((cc ^ (r & 15)) << 4));
            // rows past M fall outside rC; columns past N are dropped here.
            // Non-temporal stores (cache-policy bit nt): the output is not
            // read again by this kernel, and writing it through while the
            // matrix cores are busy keeps it from sitting dirty in the caches
            // and being written back under the next kernel's loads.
            const uint32_t off = col < P.N ? (uint32_t)((size_t)(wrow0 + r - m0) * N2 + (size_t)col * 2) : kOOB;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v),
                                                   rC, off, 0, kStoreNT);
        }
    };

    // ---- single adapter, r <= 32, aligned rank-side operands: every epilogue
    // load (the column-side fragments, the wave's 128 rows of S / dS and, for
    // B3, its keep words) is issued before any of them is used, so their
    // latencies overlap instead of adding up band by band.
    // The fast epilogue for one adapter item `it` covering all of the wave's
    // rows (r <= 32, a multiple of 8, 16-byte aligned rank-side matrix).
    auto fast_epilogue = [&](const ExtItem &it) {
        {
            // FAST == 2 (r <= 16): one 32-deep MFMA per output tile carries both
            // halves of the fp32 row side -- K slots 0-15 hold the hi parts of
            // ranks 0-15, slots 16-31 the lo parts -- against the column side's
            // ranks 0-15 repeated in both halves.  Lanes of K groups 2, 3 then
            // address the ranks of groups 0, 1.
            constexpr bool pack = FAST >= 2;
            const int lgr = pack ? (lg & 1) : lg;
            const __amdgpu_buffer_rsrc_t rW = ext_rsrc<EPI>(P, it, wcol0);
            const lds_char *pf = (const lds_char *)smem + NST * STAGE_BYTES;
            if constexpr (PF) __syncthreads();  // every wave's prefetch landed (K = 0 never waited)
            uint4 cf[NT16];
            if constexpr (PF && EPI == 2) {
                // A rows of this wave's columns, ranks 8*lgr .. +7 (zero past r)
#pragma unroll
                for (int tn = 0; tn < NT16; ++tn) {
                    const int c = wn * 128 + tn * 16 + l16;
                    cf[tn] = 8 * lgr < it.r ? *(const uint4 *)(pf + 16384 + c * it.r * 2 + lgr * 16)
                                            : make_uint4(0u, 0u, 0u, 0u);
                }
            } else if constexpr (PF) {
                const int kr = 8 * lgr + (l16 >> 2);
                const int swr = swz_w(kr);
#pragma unroll
                for (int tn = 0; tn < NT16; ++tn) {
                    const int ch = wn * 16 + 2 * tn + ((l16 & 3) >> 1);
                    const lds_char *pp = pf + 16384 + kr * 512 + ((ch ^ swr) << 4) + (l16 & 1) * 8;
                    const uint2 lo = lds_read_tr4(pp), hi = lds_read_tr4(pp + 2048);
                    cf[tn] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
#pragma unroll
                for (int tn = 0; tn < NT16; tn += 2) mfma_src_ready(cf[tn], cf[tn + 1]);
            } else if (EPI == 2) {
#pragma unroll
                for (int tn = 0; tn < NT16; ++tn)
                    cf[tn] = col_ext_frag<EPI>(P, rW, wcol0, it, wcol0 + tn * 16 + l16, 0, 16 * lgr + l16, true);
            } else {
                // B[0..32) x [wcol0, wcol0+128) through this wave's 8 KiB of LDS
                // past the stage ring (the ring holds the output staging):
                // 16-byte loads of 256-byte rows (ranks >= r and columns >= N
                // zero), then transposing reads give each lane 8 consecutive
                // ranks of one column.
                lds_char *bs = (lds_char *)smem + NST * STAGE_BYTES + wave * 8192;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int q = lane + 64 * j, rr = q >> 4, c = q & 15;
                    const uint32_t off = (rr < it.r && wcol0 + 8 * c < P.N) ? ((uint32_t)rr * (uint32_t)P.N + 8u * c) * 2u : kOOB;
                    const uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rW, off, 0, 0));
                    *(uint4 *)(bs + rr * 256 + ((c ^ swz_w(rr)) << 4)) = v;
                }
                const int kr = 8 * lgr + (l16 >> 2);
                const int swr = swz_w(kr);
#pragma unroll
                for (int tn = 0; tn < NT16; ++tn) {
                    const int ch = 2 * tn + ((l16 & 3) >> 1);
                    const lds_char *pp = bs + kr * 256 + ((ch ^ swr) << 4) + (l16 & 1) * 8;
                    const uint2 lo = lds_read_tr4(pp), hi = lds_read_tr4(pp + 1024);
                    cf[tn] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
#pragma unroll
                for (int tn = 0; tn < NT16; tn += 2) mfma_src_ready(cf[tn], cf[tn + 1]);
            }
            const int rb = 8 * lgr;
            float4 sv[NT16][2];
            if constexpr (PF) {
                // chunks 2*lgr, 2*lgr+1 of the row; the row's swizzle is (l16 >> 2)
#pragma unroll
                for (int tm = 0; tm < NT16; ++tm) {
                    const lds_char *sr = pf + (wm * 128 + tm * 16 + l16) * 64;
                    sv[tm][0] = *(const float4 *)(sr + (((2 * lgr) ^ (l16 >> 2)) << 4));
                    sv[tm][1] = *(const float4 *)(sr + (((2 * lgr + 1) ^ (l16 >> 2)) << 4));
                }
            } else {
#pragma unroll
                for (int tm = 0; tm < NT16; ++tm) {
                    const int row = wrow0 + tm * 16 + l16;
                    const uint32_t off = (row < P.M && rb < it.r) ? (uint32_t)((tm * 16 + l16) * P.RS + rb) * 4u : kOOB;
                    sv[tm][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rS, off, 0, 0));
                    sv[tm][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rS, off == kOOB ? kOOB : off + 16, 0, 0));
                }
            }
            uint32_t kwv[NT16][NT16 / 2];
            if (PF && EPI == 2) {
                const bool has_keep = P.keep != nullptr;
#pragma unroll
                for (int tm = 0; tm < NT16; ++tm) {
                    const uint4 w4 = has_keep ? *(const uint4 *)(pf + 24576 + (wm * 128 + tm * 16 + l16) * 32 + wn * 16)
                                              : make_uint4(~0u, ~0u, ~0u, ~0u);
                    kwv[tm][0] = w4.x;
                    kwv[tm][1] = w4.y;
                    kwv[tm][2] = w4.z;
                    kwv[tm][3] = w4.w;
                }
            } else if (EPI == 2) {
                const bool has_keep = P.keep != nullptr;
                const __amdgpu_buffer_rsrc_t rK = make_rsrc(has_keep ? P.keep + (size_t)min(wrow0, P.M) * P.KW : P.keep,
                                                            has_keep ? (uint64_t)max(P.M - wrow0, 0) * (uint64_t)P.KW * 4u : 0u);
                // the wave's 128 columns are 4 consecutive mask words of each row:
                // one 16-byte load per row (the host picks this path only when
                // rows of words are 16-byte aligned; words past the row's end
                // only govern columns that are never stored)
#pragma unroll
                for (int tm = 0; tm < NT16; ++tm) {
                    const uint32_t off = has_keep ? (uint32_t)((tm * 16 + l16) * P.KW + (wcol0 >> 5)) * 4u : kOOB;
                    const uint4 w4 = has_keep ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rK, off, 0, 0))
                                              : make_uint4(~0u, ~0u, ~0u, ~0u);
                    kwv[tm][0] = w4.x;
                    kwv[tm][1] = w4.y;
                    kwv[tm][2] = w4.z;
                    kwv[tm][3] = w4.w;
                }
            }
#pragma unroll
            for (int tm = 0; tm < NT16; ++tm) {
                float v[8] = {sv[tm][0].x, sv[tm][0].y, sv[tm][0].z, sv[tm][0].w,
                              sv[tm][1].x, sv[tm][1].y, sv[tm][1].z, sv[tm][1].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] *= it.scale;
                uint4 hi, lo;
                if constexpr (pack)
                    hi = split_frag_half(v, lg >= 2);
                else
                    split_frag(v, hi, lo);
                if (EPI == 1) {
                    if constexpr (pack) {
                        mfma_src_ready(hi);
#pragma unroll
                        for (int tn = 0; tn < NT16; ++tn) mfma16x16x32_inplace(acc[tm][tn], cf[tn], hi);
                    } else {
                        mfma_src_ready(hi, lo);
#pragma unroll
                        for (int tn = 0; tn < NT16; ++tn) {
                            mfma16x16x32_inplace(acc[tm][tn], cf[tn], hi);
                            mfma16x16x32_inplace(acc[tm][tn], cf[tn], lo);
                        }
                    }
                } else {
                    f32x4_t acc2[NT16];
#pragma unroll
                    for (int tn = 0; tn < NT16; ++tn) {
                        acc2[tn] = mfma16x16x32(cf[tn], hi, f32x4_t{0.f, 0.f, 0.f, 0.f});
                        if constexpr (!pack) acc2[tn] = mfma16x16x32(cf[tn], lo, acc2[tn]);
                    }
                    // Rows past M and columns past N are staged too; the flush
                    // drops them.  A clear keep bit turns the LoRA term into +0
                    // (AND with a sign-extended bit: no compare or select).
#pragma unroll
                    for (int tn = 0; tn < NT16; ++tn) {
                        const uint32_t kw = kwv[tm][tn >> 1] >> (((tn & 1) << 4) + 4 * lg);
                        float x[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t keep = (uint32_t)((int32_t)(kw << (31 - e)) >> 31);
                            x[e] = acc[tm][tn][e] + __uint_as_float(__float_as_uint(acc2[tn][e]) & keep);
                        }
                        c_put(tm, tn, x[0], x[1], x[2], x[3]);
                    }
                }
            }
            if (EPI == 1) {
                mfma_drain();
#pragma unroll
                for (int tm = 0; tm < NT16; ++tm) {
#pragma unroll
                    for (int tn = 0; tn < NT16; ++tn) {
                        const f32x4_t a4 = acc[tm][tn];
                        c_put(tm, tn, a4[0], a4[1], a4[2], a4[3]);
                    }
                }
            }
        }
        c_flush();
    };
    if constexpr (FAST && EPI != 0 && !MULTI) {
        ExtItem it;
        get_item<EPI, MULTI>(P, 0, it);
        fast_epilogue(it);
        return;
    } else {
    // ---- B3, A staged in LDS (plan_tile_items).  After the K loop the ring
    // holds: [0, 32 KiB) the output staging, 8 KiB per wave (two 16-row
    // bands); slabs of 64 ranks at 32, 64 and 96 KiB, the first item's ranks
    // 0..63 already past the ring.  The wave runs its 16-row bands in order:
    // the next band's S / dS rows and mask words are loaded while the current
    // band's rank-deep MFMAs run, its rank chunks (at most four) come from the
    // slabs, the masked sum is staged and its 16 rows are stored at once.
    if constexpr (EPI == 2 && FAST == 0) {
        if (lds_epi) {
            const uint32_t slab_at[4] = {(uint32_t)(NST * STAGE_BYTES), 32768u, 65536u, 98304u};
            __syncthreads();  // every wave is done with the ring; slab 0 landed everywhere
            if (ti.rp[0] > 64) slab_dma(ti.it[0], 64, smem_lds + slab_at[1]);
            if (ti.n == 2) {
                slab_dma(ti.it[1], 0, smem_lds + slab_at[2]);
                if (ti.rp[1] > 64) slab_dma(ti.it[1], 64, smem_lds + slab_at[3]);
            }
            // A band's rank chunks: those of each item its 16 rows meet, item 0's
            // first (rows outside an item read zeros, so the band sums them all).
            // Up to four chunks come from registers loaded during the previous
            // band; a band meeting both items may have up to four more, loaded
            // when needed.
            auto band_nc0 = [&](int tm) {
                const int b0 = wrow0 + 16 * tm, b1 = min(b0 + 16, P.M);
                return (b0 < ti.it[0].hi && b1 > ti.it[0].lo) ? ti.rp[0] >> 5 : 0;
            };
            auto band_nsl = [&](int tm, int nc0) {
                const int b0 = wrow0 + 16 * tm, b1 = min(b0 + 16, P.M);
                return nc0 + ((ti.n == 2 && b0 < ti.it[1].hi && b1 > ti.it[1].lo) ? ti.rp[1] >> 5 : 0);
            };
            const bool has_keep = P.keep != nullptr;
            const __amdgpu_buffer_rsrc_t rK = make_rsrc(has_keep ? P.keep + (size_t)min(wrow0, P.M) * P.KW : P.keep,
                                                        has_keep ? (uint64_t)max(P.M - wrow0, 0) * (uint64_t)P.KW * 4u : 0u);
            // dS of band tm, chunk j: ranks rr0 + 8 (lane / 16) .. +7 of the lane's
            // row, as 8 fp32 values, or (split rows given) as the 8 hi and the 8
            // lo bf16 of s*dS, bit-cast into f[0] and f[1]
            const bool presplit = P.dss != nullptr;
            const __amdgpu_buffer_rsrc_t rD = make_rsrc(presplit ? P.dss + (size_t)min(wrow0, P.M) * P.dss_ld : P.dss,
                                                        presplit ? (uint64_t)max(P.M - wrow0, 0) * (uint64_t)P.dss_ld * 2u : 0u);
            auto load_slot = [&](int tm, int j, int nc0, float4 (&f)[2]) {
                const bool second = j >= nc0;
                const ExtItem &it = second ? ti.it[1] : ti.it[0];
                const int rb = 32 * (second ? j - nc0 : j) + 8 * lg;
                const int row = wrow0 + tm * 16 + l16;
                const bool ok = row >= it.lo && row < it.hi && rb < it.r;
                if (presplit) {
                    const int nbt = (it.r + 15) >> 4;
                    const int rpa = 16 * (nbt <= 1 ? 1 : nbt <= 2 ? 2 : nbt <= 4 ? 4 : 8);
                    const uint32_t base = (uint32_t)((tm * 16 + l16) * P.dss_ld + rb) * 2u;
                    f[0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rD, ok ? base : kOOB, 0, 0));
                    f[1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          rD, ok ? base + (uint32_t)rpa * 2u : kOOB, 0, 0));
                    return;
                }
                const uint32_t off = ok ? (uint32_t)((tm * 16 + l16) * P.RS + rb) * 4u : kOOB;
                f[0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rS, off, 0, 0));
                f[1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rS, ok ? off + 16u : kOOB, 0, 0));
            };
            // chunk 0 of bands 0..3 is loaded before the slabs are waited for
            // (one round trip to memory for them), that of band tm + 4 once
            // band tm's first MFMAs have read its slot (four bands ahead);
            // chunks 1..3 and the mask words of a band are loaded during the
            // band before (the mask words are needed only after its MFMAs)
            float4 rf0[4][2], rfx[2][3][2];
            uint4 kw[2];
            auto load_head = [&](int tm) {
                const int nc0 = band_nc0(tm), nsl = band_nsl(tm, nc0);
                if (nsl > 0) load_slot(tm, 0, nc0, rf0[tm & 3]);
            };
            auto load_tail = [&](int tm, int slot) {
                const int nc0 = band_nc0(tm), nsl = band_nsl(tm, nc0);
#pragma unroll
                for (int j = 1; j < 4; ++j)
                    if (j < nsl) load_slot(tm, j, nc0, rfx[slot][j - 1]);
                kw[slot] = has_keep ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                 rK, (uint32_t)((tm * 16 + l16) * P.KW + (wcol0 >> 5)) * 4u, 0, 0))
                                    : make_uint4(~0u, ~0u, ~0u, ~0u);
            };
            const int swl = (l16 >> 1) & 7;
            // rank-deep MFMAs of chunk j (the row side in f) into acc2
            auto mfma_slot = [&](int j, int nc0, const float4 (&f)[2], f32x4_t (&acc2)[NT16], auto first_c) {
                const bool second = j >= nc0;
                const int rr0 = 32 * (second ? j - nc0 : j);
                uint4 hi, lo;
                if (presplit) {
                    hi = __builtin_bit_cast(uint4, f[0]);
                    lo = __builtin_bit_cast(uint4, f[1]);
                } else {
                    const float sc = second ? ti.it[1].scale : ti.it[0].scale;
                    float v[8] = {f[0].x, f[0].y, f[0].z, f[0].w, f[1].x, f[1].y, f[1].z, f[1].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] *= sc;
                    split_frag(v, hi, lo);
                }
                const int q = ((rr0 >> 5) & 1) * 4 + lg;  // 8-rank chunk inside the slab
                const lds_char *sb = (const lds_char *)smem + slab_at[(second ? 2 : 0) + (rr0 >> 6)];
                uint4 cf[NT16];
#pragma unroll
                for (int tn = 0; tn < NT16; ++tn) {
                    const int c = wn * 128 + tn * 16 + l16;
                    cf[tn] = *(const uint4 *)(sb + c * 128 + ((q ^ swl) << 4));
                }
                // the band's accumulators stay in VGPRs (the AGPRs hold the
                // product's tiles): no copies in and out around each chunk; the
                // hi and lo MFMAs of one accumulator are 8 MFMAs apart
                mfma_src_ready(hi, lo);
#pragma unroll
                for (int tn = 0; tn < NT16; ++tn) {
                    if constexpr (decltype(first_c)::value) mfma16x16x32_vfirst(acc2[tn], cf[tn], hi);
                    else mfma16x16x32_vacc(acc2[tn], cf[tn], hi);
                }
#pragma unroll
                for (int tn = 0; tn < NT16; ++tn) mfma16x16x32_vacc(acc2[tn], cf[tn], lo);
            };
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) load_head(tm);
            load_tail(0, 0);
            wait_vmcnt<0>();
            __syncthreads();  // the slabs landed
            lds_char *stg = (lds_char *)smem + wave * 8192;
#pragma unroll
            for (int tm = 0; tm < NT16; ++tm) {
                const int cur = tm & 1;
                if (tm + 1 < NT16) load_tail(tm + 1, cur ^ 1);
                const int nc0 = band_nc0(tm), nsl = band_nsl(tm, nc0);
                f32x4_t acc2[NT16];
#pragma unroll
                for (int tn = 0; tn < NT16; ++tn) acc2[tn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                // the first chunk's MFMAs start the accumulators (zero above
                // only for a band with no chunk)
                if (nsl > 0) mfma_slot(0, nc0, rf0[tm & 3], acc2, T_{});
                if (tm + 4 < NT16) load_head(tm + 4);
#pragma unroll
                for (int j = 1; j < 4; ++j)
                    if (j < nsl) mfma_slot(j, nc0, rfx[cur][j - 1], acc2, F_{});
                for (int j = 4; j < nsl; ++j) {  // a band meeting both items
                    float4 f[2];
                    load_slot(tm, j, nc0, f);
                    mfma_slot(j, nc0, f, acc2, F_{});
                }
                mfma_drain();  // the band MFMAs' results are read below
                // masked sum into the band's staging rows (rows past M and
                // columns past N are staged too; the stores drop them)
                lds_char *sbnd = stg + (tm & 1) * 4096;
                const uint4 k4 = kw[cur];
#pragma unroll
                for (int tn = 0; tn < NT16; ++tn) {
                    const uint32_t w = (tn >> 1) == 0 ? k4.x : (tn >> 1) == 1 ? k4.y : (tn >> 1) == 2 ? k4.z : k4.w;
                    const uint32_t kwb = w >> (((tn & 1) << 4) + 4 * lg);
                    float x[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t keep = (uint32_t)((int32_t)(kwb << (31 - e)) >> 31);
                        x[e] = acc[tm][tn][e] + __uint_as_float(__float_as_uint(acc2[tn][e]) & keep);
                    }
                    const int ch = (2 * tn + (lg >> 1)) ^ l16;
                    *(uint2 *)(sbnd + l16 * 256 + ch * 16 + (lg & 1) * 8) =
                        make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
                }
                // the band's 16 rows: 4 stores of 4 whole 256-byte rows per wave
                const int cc = lane & 15;
                const int col = wcol0 + cc * 8;
#pragma unroll
                for (int it4 = 0; it4 < 4; ++it4) {
                    const int rr = it4 * 4 + (lane >> 4);
                    const uint4 v = *(const uint4 *)(sbnd + rr * 256 + ((cc ^ rr) << 4));
                    const uint32_t off = col < P.N ? (uint32_t)((size_t)(wrow0 + tm * 16 + rr - m0) * N2 + (size_t)col * 2) : kOOB;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, v),
                                                           rC, off, 0, kStoreNT);
                }
            }
            return;
        }
    }
    // mixed adapters: the wave's first segment, found once
    const int wseg = MULTI ? first_segment(P, wrow0) : 0;
    // B3 with mixed adapters: a wave whose rows all lie in one segment (wave-
    // uniform; no barrier follows in any path) takes the fast epilogue when
    // that adapter meets its conditions, else the single-adapter band path
    // below with this segment's item
    bool wave_one_seg = false;
    ExtItem wit;
    if constexpr (MULTI && EPI == 2) {
        wave_one_seg = wrow0 < P.M && wseg < P.nseg && get_item<EPI, MULTI>(P, wseg, wit) &&
                       wit.lo <= wrow0 && wit.hi >= min(wrow0 + 128, P.M);
        if (wave_one_seg && P.multi_fast && wit.r <= 32 && (wit.r & 7) == 0 && (((uintptr_t)wit.w) & 15) == 0) {
            fast_epilogue(wit);
            return;
        }
    }

    // ---- F2 (general path): alpha * S * B accumulated into acc
    if (EPI == 1) {
        int s_begin = 0, s_end = 1;
        if (MULTI) {
            s_begin = wseg;
            s_end = P.nseg;
        }
        for (int s = s_begin; s < s_end; ++s) {
            if (MULTI && P.seg_off[s] >= (int64_t)(wrow0 + 128)) break;
            ExtItem it;
            if (!get_item<EPI, MULTI>(P, s, it)) continue;
            if (it.hi <= wrow0 || it.lo >= wrow0 + 128) continue;
            const bool rvec = svec && (it.r & 7) == 0;
            const __amdgpu_buffer_rsrc_t rW = ext_rsrc<EPI>(P, it, wcol0);
            // B rows 16-byte aligned: stage ranks rr0 .. rr0+31 of the wave's
            // 128 columns through its 8 KiB past the stage ring and read them
            // back transposed (as the fast epilogue does); else 2-byte loads
            const bool bstage = (P.N & 7) == 0 && (((uintptr_t)it.w) & 15) == 0;
            for (int rr0 = 0; rr0 < it.r; rr0 += 32) {
                // B's staging loads, then the row side of all 8 bands (the
                // form chosen once, outside the band loop, so each band's
                // loads do not wait on the other form's), then B's LDS
                // writes: the chunk waits for one round trip to memory
                lds_char *bs = (lds_char *)smem + NST * STAGE_BYTES + wave * 8192;
                uint4 bv[8];
                if (bstage) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int q = lane + 64 * j, rr = q >> 4, c = q & 15;
                        const uint32_t off = (rr0 + rr < it.r && wcol0 + 8 * c < P.N)
                            ? ((uint32_t)(rr0 + rr) * (uint32_t)P.N + 8u * c) * 2u : kOOB;
                        bv[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rW, off, 0, 0));
                    }
                }
                float sv[NT16][8];
                if (rvec) {
#pragma unroll
                    for (int tm = 0; tm < NT16; ++tm) row_ext_load(P, rS, wrow0, it, wrow0 + tm * 16 + l16, rr0, lane, true, sv[tm]);
                } else {
#pragma unroll
                    for (int tm = 0; tm < NT16; ++tm) row_ext_load(P, rS, wrow0, it, wrow0 + tm * 16 + l16, rr0, lane, false, sv[tm]);
                }
                uint4 cf[NT16];
                if (bstage) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int q = lane + 64 * j, rr = q >> 4, c = q & 15;
                        *(uint4 *)(bs + rr * 256 + ((c ^ swz_w(rr)) << 4)) = bv[j];
                    }
                    const int kr = 8 * lg + (l16 >> 2);
                    const int swr = swz_w(kr);
#pragma unroll
                    for (int tn = 0; tn < NT16; ++tn) {
                        const int ch = 2 * tn + ((l16 & 3) >> 1);
                        const lds_char *pp = bs + kr * 256 + ((ch ^ swr) << 4) + (l16 & 1) * 8;
                        const uint2 lo = lds_read_tr4(pp), hi = lds_read_tr4(pp + 1024);
                        cf[tn] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                    }
                } else {
#pragma unroll
                    for (int tn = 0; tn < NT16; ++tn) cf[tn] = col_ext_frag<EPI>(P, rW, wcol0, it, wcol0 + tn * 16 + l16, rr0, lane, false);
                }
#pragma unroll
                for (int tn = 0; tn < NT16; tn += 2) mfma_src_ready(cf[tn], cf[tn + 1]);
#pragma unroll
                for (int tm = 0; tm < NT16; ++tm) {
                    uint4 hi, lo;
                    row_ext_split(it, sv[tm], hi, lo);
                    mfma_src_ready(hi, lo);
#pragma unroll
                    for (int tn = 0; tn < NT16; ++tn) {
                        mfma16x16x32_inplace(acc[tm][tn], cf[tn], hi);
                        mfma16x16x32_inplace(acc[tm][tn], cf[tn], lo);
                    }
                }
            }
        }
        mfma_drain();
    }

    // ---- B3, single adapter with r <= 64: the column-side A fragments (one
    // or two rank chunks of 32) are the same for every 16-row band, loaded once
    // Mixed adapters, a wave whose rows meet exactly two segments of ranks <=
    // 32: the same two fragment slots hold the first item's ranks 0..31 and
    // the second item's; rows outside an item read zeros, so each band adds
    // both terms.  Both items and their fragments are looked up once, not per
    // band.
    uint4 cf1[2][NT16];
    bool one_chunk = false;  // r <= 64 (the name predates the second chunk)
    ExtItem it1, it2;        // items of fragment slots 0 and 1
    int rk2 = 32;            // first rank of slot 1
    bool rvec1 = false, rvec2 = false;
    if (EPI == 2 && (!MULTI || wave_one_seg)) {
        if (MULTI) it1 = wit;
        else get_item<EPI, MULTI>(P, 0, it1);
        one_chunk = it1.r <= 64;
        it2 = it1;
        rvec1 = rvec2 = svec && (it1.r & 7) == 0;
    }
    if constexpr (MULTI && EPI == 2) {
        if (!wave_one_seg && wrow0 < P.M && wseg < P.nseg) {
            int s2 = wseg + 1;
            while (s2 < P.nseg && P.seg_off[s2 + 1] <= P.seg_off[s2]) ++s2;  // skip empty segments
            if (s2 < P.nseg && get_item<EPI, MULTI>(P, wseg, it1) && get_item<EPI, MULTI>(P, s2, it2) &&
                it1.lo <= wrow0 && it1.hi == it2.lo && it2.hi >= min(wrow0 + 128, P.M) && it1.r <= 32 &&
                it2.r <= 32) {
                one_chunk = true;
                rk2 = 0;
                rvec1 = svec && (it1.r & 7) == 0;
                rvec2 = svec && (it2.r & 7) == 0;
            }
        }
    }
    if (EPI == 2 && one_chunk) {
        const bool avec1 = (it1.r & 7) == 0 && (((uintptr_t)it1.w) & 15) == 0;
        const bool avec2 = (it2.r & 7) == 0 && (((uintptr_t)it2.w) & 15) == 0;
        const __amdgpu_buffer_rsrc_t rW1 = ext_rsrc<EPI>(P, it1, wcol0);
        const __amdgpu_buffer_rsrc_t rW2 = ext_rsrc<EPI>(P, it2, wcol0);
#pragma unroll
        for (int tn = 0; tn < NT16; ++tn) {
            cf1[0][tn] = col_ext_frag<EPI>(P, rW1, wcol0, it1, wcol0 + tn * 16 + l16, 0, lane, avec1);
            cf1[1][tn] = col_ext_frag<EPI>(P, rW2, wcol0, it2, wcol0 + tn * 16 + l16, rk2, lane, avec2);
        }
    }

    // ---- output (B3 adds the masked rank-deep term one 16-row band at a time)
    const bool has_keep = EPI == 2 && P.keep != nullptr;
    const __amdgpu_buffer_rsrc_t rK = make_rsrc(has_keep ? P.keep + (size_t)min(wrow0, P.M) * P.KW : P.keep,
                                                has_keep ? (uint64_t)max(P.M - wrow0, 0) * (uint64_t)P.KW * 4u : 0u);
#pragma unroll
    for (int tm = 0; tm < NT16; ++tm) {
        const int row = wrow0 + tm * 16 + l16;
        f32x4_t acc2[NT16];
        uint4 kw4 = make_uint4(~0u, ~0u, ~0u, ~0u);
        if (EPI == 2) {
            // the band's mask words (the wave's 128 columns are 4 words of each
            // row), issued ahead of its rank-deep loads
            if (has_keep && P.keep16)
                kw4 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rK, (uint32_t)((tm * 16 + l16) * P.KW + (wcol0 >> 5)) * 4u, 0, 0));
#pragma unroll
            for (int tn = 0; tn < NT16; ++tn) acc2[tn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (one_chunk) {
                // both slots' row-side loads first; one item with r <= 32
                // leaves slot 1 all zeros (out-of-range offsets)
                uint4 hi0, lo0, hi1, lo1;
                row_ext_frags(P, rS, wrow0, it1, row, 0, lane, rvec1, hi0, lo0);
                row_ext_frags(P, rS, wrow0, it2, row, rk2, lane, rvec2, hi1, lo1);
#pragma unroll
                for (int tn = 0; tn < NT16; ++tn) {
                    acc2[tn] = mfma16x16x32(cf1[0][tn], hi0, acc2[tn]);
                    acc2[tn] = mfma16x16x32(cf1[0][tn], lo0, acc2[tn]);
                }
                if (it1.r > 32 || rk2 == 0) {
#pragma unroll
                    for (int tn = 0; tn < NT16; ++tn) {
                        acc2[tn] = mfma16x16x32(cf1[1][tn], hi1, acc2[tn]);
                        acc2[tn] = mfma16x16x32(cf1[1][tn], lo1, acc2[tn]);
                    }
                }
            } else {
                const int band0 = wrow0 + tm * 16;
                int s_begin = 0, s_end = 1;
                if (MULTI && !wave_one_seg) {
                    // first segment ending past the band, stepping on from the wave's
                    s_begin = wseg;
                    while (s_begin < P.nseg && P.seg_off[s_begin + 1] <= (int64_t)band0) ++s_begin;
                    s_end = P.nseg;
                }
                for (int s = s_begin; s < s_end; ++s) {
                    ExtItem it;
                    if (MULTI && wave_one_seg) {
                        it = wit;  // the wave's one segment, looked up once
                    } else {
                        if (MULTI && P.seg_off[s] >= (int64_t)(band0 + 16)) break;
                        if (!get_item<EPI, MULTI>(P, s, it)) continue;
                    }
                    if (it.hi <= band0 || it.lo >= band0 + 16) continue;
                    const bool rvec = svec && (it.r & 7) == 0;
                    const bool avec = (it.r & 7) == 0 && (((uintptr_t)it.w) & 15) == 0;
                    const __amdgpu_buffer_rsrc_t rW = ext_rsrc<EPI>(P, it, wcol0);
                    for (int rr0 = 0; rr0 < it.r; rr0 += 32) {
                        uint4 hi, lo;
                        row_ext_frags(P, rS, wrow0, it, row, rr0, lane, rvec, hi, lo);
#pragma unroll
                        for (int tn = 0; tn < NT16; ++tn) {
                            const uint4 cf = col_ext_frag<EPI>(P, rW, wcol0, it, wcol0 + tn * 16 + l16, rr0, lane, avec);
                            acc2[tn] = mfma16x16x32(cf, hi, acc2[tn]);
                            acc2[tn] = mfma16x16x32(cf, lo, acc2[tn]);
                        }
                    }
                }
            }
        }
        if constexpr (EPI != 2) {
            if (row < P.M) {
#pragma unroll
                for (int tn = 0; tn < NT16; ++tn) {
                    const int col = wcol0 + tn * 16 + 4 * lg;
                    if (col >= P.N) continue;
                    const f32x4_t a4 = acc[tm][tn];
                    c_put(tm, tn, a4[0], a4[1], a4[2], a4[3]);
                }
            }
            continue;
        }
        // rows past M and columns past N are staged too; the flush drops them
#pragma unroll
        for (int tn = 0; tn < NT16; ++tn) {
            float x[4];
            if (EPI == 2) {
                uint32_t kw = ~0u;
                if (has_keep) {
                    if (P.keep16) {
                        const uint32_t w = (tn >> 1) == 0 ? kw4.x : (tn >> 1) == 1 ? kw4.y : (tn >> 1) == 2 ? kw4.z : kw4.w;
                        kw = w >> (((tn & 1) << 4) + 4 * lg);
                    } else {
                        const int col = wcol0 + tn * 16 + 4 * lg;
                        kw = (row < P.M && col < P.N) ? P.keep[(size_t)row * P.KW + (col >> 5)] >> (col & 31) : 0u;
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t keep = (uint32_t)((int32_t)(kw << (31 - e)) >> 31);
                    x[e] = acc[tm][tn][e] + __uint_as_float(__float_as_uint(acc2[tn][e]) & keep);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = acc[tm][tn][e];
            }
            c_put(tm, tn, x[0], x[1], x[2], x[3]);
        }
    }
    c_flush();
    }  // general epilogue
}

// the stage ring plus 8 KiB per wave for the forward epilogue's B staging
size_t gemm_lds_bytes() { return (size_t)NST * STAGE_BYTES + 4 * 8192; }

template <bool NN, int EPI, bool MULTI, int FAST>
static hipError_t launch_gemm_t(const GemmParams &P, hipStream_t stream, const char *name) {
    const size_t lds = gemm_lds_bytes();
    const int G = P.tiles_m * P.tiles_n;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)gemm_kernel<NN, EPI, MULTI, FAST>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    (void)hipGetLastError();
    const int slot = prof_begin(name, stream);
    hipLaunchKernelGGL((gemm_kernel<NN, EPI, MULTI, FAST>), dim3(G), dim3(256), lds, stream, P);
    hipError_t e = hipGetLastError();
    prof_end(slot, stream);
    return e;
}

hipError_t launch_gemm(bool nn, int epi, const void *Arow, const void *Bcol, void *C, int M, int N,
                       int K, const float *Sx, int RS, const uint32_t *keep, int KW,
                       const AdapterSource &src, hipStream_t stream, const uint16_t *dss, int dss_ld) {
    GemmParams P{};
    P.dss = epi == 2 ? dss : nullptr;
    P.dss_ld = dss_ld;
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
    auto al16 = [](const void *q) { return ((uintptr_t)q & 15) == 0; };
    const bool fast = !multi && epi != 0 && P.ext_r <= 32 && (P.ext_r & 7) == 0 && (RS & 7) == 0 &&
                      al16(Sx) && al16(P.ext) && (epi != 2 || ((KW & 3) == 0 && al16(keep)));
    const bool pack = fast && P.ext_r <= 16 && RS <= 16;
    P.keep16 = (KW & 3) == 0 && al16(keep);
    P.multi_fast = multi && epi != 0 && (RS & 7) == 0 && al16(Sx) && (epi != 2 || ((KW & 3) == 0 && al16(keep)));
    if (nn) {
        if (epi == 0) return launch_gemm_t<true, 0, false, 0>(P, stream, "gemm_frozen_fwd");
        if (epi == 1) return multi ? launch_gemm_t<true, 1, true, 0>(P, stream, "gemm_f2_fwd_lora")
                             : pack ? launch_gemm_t<true, 1, false, 2>(P, stream, "gemm_f2_fwd_lora")
                             : fast ? launch_gemm_t<true, 1, false, 1>(P, stream, "gemm_f2_fwd_lora")
                                    : launch_gemm_t<true, 1, false, 0>(P, stream, "gemm_f2_fwd_lora");
    } else {
        if (epi == 0) return launch_gemm_t<false, 0, false, 0>(P, stream, "gemm_frozen_bwd");
        if (epi == 2) return multi ? launch_gemm_t<false, 2, true, 0>(P, stream, "gemm_b3_bwd_dx")
                             : pack ? launch_gemm_t<false, 2, false, 2>(P, stream, "gemm_b3_bwd_dx")
                             : fast ? launch_gemm_t<false, 2, false, 1>(P, stream, "gemm_b3_bwd_dx")
                                    : launch_gemm_t<false, 2, false, 0>(P, stream, "gemm_b3_bwd_dx");
    }
    return hipErrorInvalidValue;
}

hipError_t launch_gemm_cat(const void *X, const void *W, const void *A, const void *B, void *Y, float *S,
                           int M, int N, int K, int r, float alpha, hipStream_t stream) {
    GemmParams P{};
    P.Arow = (const uint16_t *)X;
    P.Bcol = (const uint16_t *)W;
    P.C = (uint16_t *)Y;
    P.M = M;
    P.N = N;
    P.K = K;
    P.tiles_m = (M + GBM - 1) / GBM;
    P.tiles_n = (N + GBN - 1) / GBN;
    P.ext = (const uint16_t *)B;
    P.ext_r = r;
    P.ext_scale = alpha;
    P.Sx = S;
    P.RS = r;
    P.catA = (const uint16_t *)A;
    P.Sout = S;
    if (P.tiles_m == 0 || P.tiles_n == 0) return hipSuccess;
    // the kernel's fixed layout: ranks 8 or 16, A and B rows in whole 16-byte pieces
    auto al16 = [](const void *q) { return ((uintptr_t)q & 15) == 0; };
    if ((r != 8 && r != 16) || !al16(A) || !al16(B) || !al16(S)) return hipErrorInvalidValue;
    return launch_gemm_t<true, 1, false, 3>(P, stream, "gemm_f2_concat_p0");
}

hipError_t launch_gemm_kext(const void *X, const void *W, void *Y, int M, int N, int K, const uint16_t *S2,
                            int kx, const void *B, int r, hipStream_t stream) {
    GemmParams P{};
    P.Arow = (const uint16_t *)X;
    P.Bcol = (const uint16_t *)W;
    P.C = (uint16_t *)Y;
    P.M = M;
    P.N = N;
    P.K = K;
    P.tiles_m = (M + GBM - 1) / GBM;
    P.tiles_n = (N + GBN - 1) / GBN;
    P.ext = (const uint16_t *)B;
    P.ext_r = r;
    P.S2 = S2;
    P.kx = kx;
    if (P.tiles_m == 0 || P.tiles_n == 0) return hipSuccess;
    return launch_gemm_t<true, 3, false, 0>(P, stream, "gemm_f2_fwd_lora");
}

}  // namespace lora
