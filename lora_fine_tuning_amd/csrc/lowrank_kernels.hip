// Low-rank (HBM-bound) kernels of the gfx950 LoRA path:
//   router      segment table -> row chunks, one adapter per chunk
//   F1          dropout mask + S = s*(keep.X)A, one pass over X
//   B1          dS = alpha*dY B^T and dB = alpha*S^T dY, one pass over dY
//   B2          dA = s*(keep.X)^T dS, one pass over X and the mask
//   reductions  deterministic fixed-order sums of the split partials
//   mask        the dropout mask alone
// The graph is split at the rank-r tensor S as the pages describe (juhe.plus
// blog on LoRAFusion, section 4.1 "graph splitting": the work before S and the
// work after S go to different kernels; S is small enough to store).  Every
// contraction here runs on MFMA 16x16x32 bf16 with fp32 accumulation; fp32
// operands (S, dS) enter as hi+lo bf16 pairs so they keep ~fp32 precision.
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace lora {

// ===========================================================================
// Router: chunk tables for the low-rank kernels (papers.chlience.com notes,
// section 5 "FusedMultiLoRA": tile-level routing by adapter id).  Each
// non-empty segment with a valid adapter is cut into runs of at most
// `rows` rows for each of up to three tables; one work-group scans the
// segments.  A table with rows == 0 is skipped.
// Chunks are ordered by the work their adapter's rank brings, heaviest first
// (rank classes of 16-rank blocks: more than 4, 3-4, 2, 1), in segment order
// within a class: a kernel whose grid is about one round of work-groups then
// starts every heavy chunk at once instead of leaving the last segments'
// chunks for a second round.  Every consumer is order-free (sums over a
// table run in table order, which is fixed by the segment table).
// ===========================================================================
struct RouterTable {
    ChunkEntry *t;
    int32_t *c;
    int rows;
    int cap;
};
struct RouterTables {
    RouterTable tab[3];
};

constexpr int kRankClasses = 4;
__device__ __forceinline__ int rank_class(int r) {  // 3 = heaviest
    const int nbt = (r + 15) >> 4;
    return nbt <= 1 ? 0 : nbt <= 2 ? 1 : nbt <= 4 ? 2 : 3;
}

__global__ __launch_bounds__(1024) void router_kernel(const int64_t *seg_off, const int32_t *seg_ad,
                                                     int nseg, int m, const lora_adapter *adapters,
                                                     int nad, int r_cap, RouterTables T, int32_t *ad_items) {
    __shared__ int sc[3][kRankClasses][1024];
    __shared__ int tot[3][kRankClasses];
    const int tid = threadIdx.x;
    // work items of each adapter in the backward table (table 1), for the
    // fused per-adapter sums of the dA kernel
    if (ad_items != nullptr)
        for (int i = tid; i < nad; i += 1024) ad_items[i] = 0;
    if (tid < 3 * kRankClasses) tot[tid / kRankClasses][tid % kRankClasses] = 0;
    // segment s: rows [lo, hi), adapter a, its rank class and chunk counts
    auto seg_info = [&](int s, int &lo, int &hi, int &a, int &cls, int (&nq)[3]) {
        lo = hi = 0;
        a = -1;
        cls = 0;
        nq[0] = nq[1] = nq[2] = 0;
        if (s >= nseg) return;
        const int64_t o0 = seg_off[s], o1 = seg_off[s + 1];
        lo = (int)max((int64_t)0, min(o0, (int64_t)m));
        hi = (int)max((int64_t)lo, min(o1, (int64_t)m));
        a = seg_ad[s];
        if (a < 0 || a >= nad || hi <= lo) return;
        const int r = adapters[a].r;
        if (r < 1 || r > r_cap) return;
        cls = rank_class(r);
#pragma unroll
        for (int j = 0; j < 3; ++j) nq[j] = T.tab[j].rows > 0 ? (hi - lo + T.tab[j].rows - 1) / T.tab[j].rows : 0;
    };
    // A table of at most 64 segments (the usual case): one wave, one lane per
    // segment, scans by lane shuffles and no work-group barrier in the scan.
    if (nseg <= 64) {
        __syncthreads();  // the ad_items reset is visible
        if (tid >= 64) return;
        int lo, hi, a, cls, nq[3];
        seg_info(tid, lo, hi, a, cls, nq);
        if (ad_items != nullptr && nq[1] > 0) atomicAdd(&ad_items[a], nq[1]);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            int incl[kRankClasses], total[kRankClasses];
#pragma unroll
            for (int c = 0; c < kRankClasses; ++c) {
                int v = c == cls ? nq[j] : 0;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const int u = __shfl_up(v, d);
                    if (tid >= d) v += u;
                }
                incl[c] = v;
                total[c] = __shfl(v, 63);
            }
            int pos = 0, all = 0;
#pragma unroll
            for (int c = kRankClasses - 1; c >= 0; --c) {  // heavier classes first
                if (c == cls) pos = all + incl[c] - nq[j];
                all += total[c];
            }
            const int rows = T.tab[j].rows;
            for (int q = 0; q < nq[j]; ++q) {
                if (pos + q < T.tab[j].cap) {
                    ChunkEntry e;
                    e.row_lo = lo + q * rows;
                    e.row_hi = min(hi, lo + (q + 1) * rows);
                    e.adapter = a;
                    e.pad = 0;
                    T.tab[j].t[pos + q] = e;
                }
            }
            if (tid == 0 && rows > 0) T.tab[j].c[0] = min(all, T.tab[j].cap);
        }
        return;
    }
    __syncthreads();
    // pass 1: chunks per table and class (integer sums: any order)
    for (int s = tid; s < nseg; s += 1024) {
        int lo, hi, a, cls, nq[3];
        seg_info(s, lo, hi, a, cls, nq);
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (nq[j] > 0) atomicAdd(&tot[j][cls], nq[j]);
        if (ad_items != nullptr && nq[1] > 0) atomicAdd(&ad_items[a], nq[1]);
    }
    __syncthreads();
    // first position of each class: the heavier classes come first
    int cbase[3][kRankClasses], carry[3][kRankClasses];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        int acc = 0;
#pragma unroll
        for (int c = kRankClasses - 1; c >= 0; --c) {
            cbase[j][c] = acc;
            acc += tot[j][c];
            carry[j][c] = 0;
        }
    }
    // pass 2: positions by a scan per table and class over the segments
    for (int base = 0; base < nseg; base += 1024) {
        int lo, hi, a, cls, nq[3];
        seg_info(base + tid, lo, hi, a, cls, nq);
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int c = 0; c < kRankClasses; ++c) sc[j][c][tid] = c == cls ? nq[j] : 0;
        __syncthreads();
        for (int d = 1; d < 1024; d <<= 1) {
            int v[3][kRankClasses];
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
                for (int c = 0; c < kRankClasses; ++c) v[j][c] = tid >= d ? sc[j][c][tid - d] : 0;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
                for (int c = 0; c < kRankClasses; ++c) sc[j][c][tid] += v[j][c];
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int rows = T.tab[j].rows;
            int cb = 0, cc = 0, incl = 0;
#pragma unroll
            for (int c = 0; c < kRankClasses; ++c)
                if (c == cls) {
                    cb = cbase[j][c];
                    cc = carry[j][c];
                    incl = sc[j][c][tid];
                }
            const int pos = cb + cc + incl - nq[j];
            for (int q = 0; q < nq[j]; ++q) {
                if (pos + q < T.tab[j].cap) {
                    ChunkEntry e;
                    e.row_lo = lo + q * rows;
                    e.row_hi = min(hi, lo + (q + 1) * rows);
                    e.adapter = a;
                    e.pad = 0;
                    T.tab[j].t[pos + q] = e;
                }
            }
#pragma unroll
            for (int c = 0; c < kRankClasses; ++c) carry[j][c] += sc[j][c][1023];
        }
        __syncthreads();
    }
    if (tid == 0)
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (T.tab[j].rows > 0) {
                int total = 0;
#pragma unroll
                for (int c = 0; c < kRankClasses; ++c) total += tot[j][c];
                T.tab[j].c[0] = min(total, T.tab[j].cap);
            }
}

static RowWork make_work(const AdapterSource &src, WorkTable tab) {
    RowWork w;
    const ChunkEntry *const tabs[3] = {src.chunks_f1, src.chunks_bwd, src.chunks_b1};
    const int32_t *const counts[3] = {src.count_f1, src.count_bwd, src.count_b1};
    w.chunks = src.table ? tabs[tab] : nullptr;
    w.chunk_count = src.table ? counts[tab] : nullptr;
    w.adapters = src.table;
    w.num_adapters = src.num_adapters;
    w.rows_per_chunk = tab == kTabF1 ? kF1Rows : kBwdRows;
    w.r_cap = src.table ? src.r_cap : src.r;
    w.single.A = (const uint16_t *)src.A;
    w.single.B = (const uint16_t *)src.B;
    w.single.dA = (uint16_t *)src.dA;
    w.single.dB = (uint16_t *)src.dB;
    w.single.r = src.r;
    w.single.alpha = src.alpha;
    w.single.p = src.p;
    return w;
}

// ===========================================================================
// F1: dropout mask + down-projection (juhe.plus blog, section 4.1, forward
// item 1: dropout and X -> S in one kernel so X is read once).
// ===========================================================================
struct F1Params {
    const uint16_t *X;
    int m, k;
    RowWork work;
    uint64_t seed, offset;
    uint32_t *keep_bits;
    float *out;  // KS == 1: S; else partials [KS][m][RS]
    int RS;
    int ksl;
    int KW;
    int r_lds;  // rows of the staged At buffer (>= every rank, multiple of 16)
    int slab;   // columns of A staged at once (multiple of kF1KSub)
    // streaming form, single adapter: also write alpha*S split into bf16 hi
    // and lo parts, row i = [hi of ranks 0..RP) | lo of ranks 0..RP), RP = s2_rp
    // (zeros past r) -- the extra K columns of the forward GEMM
    uint16_t *s2;
    int s2_rp;
};

// F1: dropout mask + down-projection (juhe.plus blog, section 4.1, forward
// item 1: dropout and X -> S in one kernel so X is read once).
// Work-group = 4 waves x 16 rows of one chunk, over one k-slice.  Lane l of a
// wave owns row (l % 16) and the 8 columns 8*(l/16).. of each 32-wide K step:
// exactly one Philox block and one MFMA A-fragment.  A is staged transposed
// in LDS (At[rr][kk]) one slab of columns at a time, and the X loads of the
// next 128-column sub-slice are in flight while the current one is hashed,
// masked and multiplied.
template <int MAXT>
__global__ __launch_bounds__(256) void f1_kernel(F1Params P) {
    extern __shared__ uint4 f1_smem[];
    uint16_t *At = (uint16_t *)f1_smem;
    const int lda = P.slab + 8;  // LDS row stride of At (elements)

    int row_lo, row_hi;
    AdapterView ad;
    if (!resolve_chunk(P.work, blockIdx.x, P.m, row_lo, row_hi, ad)) return;
    const int r = ad.r;
    const int nbt = (r + 15) >> 4;
    const int rpad = nbt * 16;
    const uint32_t T = drop_threshold(ad.p);
    const float s = drop_scale(ad.p);
    const int kb = blockIdx.y * P.ksl;
    const int ke = min(P.k, kb + P.ksl);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, li = lane & 15;
    const int row = row_lo + wave * 16 + li;
    const bool rvalid = row < row_hi;
    const uint16_t *xrow = P.X + (size_t)(rvalid ? row : row_lo) * P.k;
    const uint64_t ctr_row = P.offset + (uint64_t)(rvalid ? row : row_lo) * (uint64_t)P.k;
    const bool vecA = (r & 7) == 0 && (((uintptr_t)ad.A) & 15) == 0;

    f32x4_t acc[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto load_x = [&](int k0, uint4 (&xv)[4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c0 = k0 + 32 * t + 8 * g;
            xv[t] = (rvalid && c0 < ke) ? *(const uint4 *)(xrow + c0) : make_uint4(0, 0, 0, 0);
        }
    };

    for (int s0 = kb; s0 < ke; s0 += P.slab) {
        const int s1 = min(ke, s0 + P.slab);
        const int cols = s1 - s0;
        __syncthreads();
        if (vecA) {
            const int vpr = r >> 3;  // 16-byte vectors per A row
            for (int idx = tid; idx < cols * vpr; idx += 256) {
                const int kk = idx / vpr, v = idx - kk * vpr;
                const uint4 a = *(const uint4 *)(ad.A + (size_t)(s0 + kk) * r + 8 * v);
                const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    At[(8 * v + e) * lda + kk] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
            }
            for (int idx = tid; idx < (rpad - r) * cols; idx += 256) {
                const int rr = r + idx / cols, kk = idx % cols;
                At[rr * lda + kk] = 0;
            }
        } else {
            for (int idx = tid; idx < cols * rpad; idx += 256) {
                const int kk = idx / rpad, rr = idx - kk * rpad;
                uint16_t v = 0;
                if (rr < r) v = ad.A[(size_t)(s0 + kk) * r + rr];
                At[rr * lda + kk] = v;
            }
        }
        // zero the tail of a ragged slab so every 128-column step reads defined values
        for (int idx = tid; idx < rpad * (P.slab - cols); idx += 256) {
            const int rr = idx / (P.slab - cols), kk = cols + idx % (P.slab - cols);
            At[rr * lda + kk] = 0;
        }
        __syncthreads();

        uint4 xa[4], xb[4];
        load_x(s0, xa);
        for (int k0 = s0; k0 < s1; k0 += kF1KSub) {
            load_x(k0 + kF1KSub, xb);  // next sub-slice (columns past ke read as zero)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int c0 = k0 + 32 * t + 8 * g;
                uint32_t byte = 0;
                if (rvalid && c0 < ke) byte = (T == 0) ? 0xFFu : keep_byte(ctr_row + (uint64_t)c0, P.seed, T);
                const uint4 xm = apply_keep(xa[t], byte);
                if (P.keep_bits != nullptr) {
                    uint32_t w = byte << (8 * g);
                    w |= (uint32_t)__shfl_xor((int)w, 16);
                    w |= (uint32_t)__shfl_xor((int)w, 32);
                    if (g == 0 && rvalid && k0 + 32 * t < ke)
                        P.keep_bits[(size_t)row * P.KW + ((k0 + 32 * t) >> 5)] = w;
                }
#pragma unroll
                for (int bt = 0; bt < MAXT; ++bt) {
                    if (bt < nbt) {
                        const uint4 bf = *(const uint4 *)&At[(bt * 16 + li) * lda + (k0 - s0) + 32 * t + 8 * g];
                        acc[bt] = mfma16x16x32(xm, bf, acc[bt]);
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) xa[t] = xb[t];
        }
    }

    float *out = P.out + (size_t)blockIdx.y * (size_t)P.m * P.RS;
#pragma unroll
    for (int bt = 0; bt < MAXT; ++bt) {
        if (bt < nbt) {
            const int col = bt * 16 + li;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int orow = row_lo + wave * 16 + 4 * g + v;
                if (orow < row_hi && col < P.RS) out[(size_t)orow * P.RS + col] = col < r ? acc[bt][v] * s : 0.f;
            }
        }
    }
    for (int col = rpad + li; col < P.RS; col += 16) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int orow = row_lo + wave * 16 + 4 * g + v;
            if (orow < row_hi) out[(size_t)orow * P.RS + col] = 0.f;
        }
    }
}

// ----- F1 streaming form (ranks <= 32 per launch slice; larger ranks in rank
// tiles of 32).  Work-group = 16 rows of a chunk over all of k, so S leaves
// the kernel finished (no split-k partials, no second launch).  Its 4 waves
// take 4 consecutive ranges of k in 128-column units (4 waves with longer
// ranges measured no slower than 8 at rank 16 and faster at 64).  Lane l owns row
// (l % 16) and columns 8*(l/16) .. +7 of each 32-column step: one Philox
// block, one keep byte, one MFMA row-side fragment.  Per unit, each wave
// copies the 128 rows of A it needs (k-major, rl bf16 per row) into a
// private LDS slab and reads its
// rank-side fragments back with transposing LDS reads; the next unit's A and
// X loads are in flight while the current unit is hashed, masked and
// multiplied.  The waves' partial S meet in LDS and are summed in wave order.
constexpr int F1S_WAVES = 4;
constexpr int F1S_UNIT = 128;  // k columns per unit (4 MFMA steps)

template <int MAXT>  // rank blocks of 16: rl = 16 * MAXT
__global__ __launch_bounds__(64 * F1S_WAVES) void f1s_kernel(F1Params P) {
    constexpr int RL = 16 * MAXT;
    constexpr int SLAB = F1S_UNIT * RL * 2;  // bytes of A per unit
    constexpr int NAV = SLAB / (16 * 64);    // 16-byte A loads per lane per unit
    extern __shared__ uint4 f1s_smem[];
    lds_char *smem = (lds_char *)f1s_smem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;

    int row_lo, row_hi;
    AdapterView ad;
    if (!resolve_chunk(P.work, blockIdx.x >> 2, P.m, row_lo, row_hi, ad)) return;
    row_lo += 16 * (blockIdx.x & 3);
    if (row_lo >= row_hi) return;
    row_hi = min(row_hi, row_lo + 16);
    const int r = ad.r;
    // rank tile blockIdx.y: ranks r0 .. r0+RL-1 of S (ranks above 32 take
    // several tiles; each reads X again and only the first writes the mask)
    const int r0 = blockIdx.y * RL;
    const int ncol = min(RL, P.RS - r0);  // S columns this tile writes
    if (r0 >= r) {
        // no ranks of this adapter here: the tile's S (and hi / lo) columns are zero
        for (int i = tid; i < 16 * RL; i += 64 * F1S_WAVES) {
            const int rr = i / RL, cl = i % RL;
            if (row_lo + rr >= row_hi) continue;
            if (cl < ncol) P.out[(size_t)(row_lo + rr) * P.RS + r0 + cl] = 0.f;
            if (P.s2 != nullptr && r0 + cl < P.s2_rp) {
                uint16_t *q = P.s2 + (size_t)(row_lo + rr) * (2 * P.s2_rp) + r0 + cl;
                q[0] = 0;
                q[P.s2_rp] = 0;
            }
        }
        return;
    }
    const uint32_t T = drop_threshold(ad.p);
    const uint32_t tm1x2 = ((T - 1u) & 0xFFFFu) * 0x00010001u;  // used only when T >= 1
    const float s = drop_scale(ad.p);

    // X rows row_lo .. row_hi-1 as one buffer: lanes of missing rows and
    // columns past the wave's range read zeros (host guarantees 16*k*2 < 2^31)
    const int nrows = row_hi - row_lo;
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(P.X + (size_t)row_lo * P.k, (size_t)nrows * P.k * 2);
    const uint32_t xrow_off = (uint32_t)l16 * (uint32_t)P.k * 2u;
    const int row = row_lo + l16;
    const bool rvalid = l16 < nrows;
    // Philox block of the lane's first element in a step starting at column c:
    // (offset + row*k + c + 8g) / 8, all terms multiples of 8
    const uint64_t blk0 = (P.offset >> 3) + (uint64_t)(rvalid ? row : row_lo) * (uint64_t)(P.k >> 3) + (uint64_t)g;

    const int kq = ((P.k + F1S_WAVES * F1S_UNIT - 1) / (F1S_WAVES * F1S_UNIT)) * F1S_UNIT;
    const int kb = wave * kq, ke = min(P.k, kb + kq);
    const int nu = ke > kb ? (ke - kb + F1S_UNIT - 1) / F1S_UNIT : 0;
    // A slabs per wave: two for RL = 16; one for RL = 32 (the next unit's A is
    // stored after this unit's last read of it -- LDS accesses of a wave are
    // performed in order), so two work-groups fit a CU
    constexpr int NSLAB = MAXT == 1 ? 2 : 1;
    lds_char *slab0 = smem + wave * NSLAB * SLAB;
    const bool avec = (r & 7) == 0 && (((uintptr_t)ad.A) & 15) == 0;
    // A rows below ke (rows at or past ke read as zero)
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(ad.A, (size_t)max(ke, 0) * r * 2);

    f32x4_t acc[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto load_x = [&](int c, uint4 (&xv)[4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c0 = c + 32 * t + 8 * g;
            const uint32_t off = c0 < ke ? xrow_off + (uint32_t)c0 * 2u : kOOB;
            xv[t] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rX, off, 0, 0));
        }
    };
    // 16-byte vector q of the slab: k row q / (RL/8), ranks r0 + 8 (q % (RL/8)) .. +7
    auto load_a = [&](int c, uint4 (&av)[NAV]) {
#pragma unroll
        for (int j = 0; j < NAV; ++j) {
            const int q = lane + 64 * j, kk = q / (RL / 8), v = q % (RL / 8);
            const uint32_t off = r0 + 8 * v < r ? ((uint32_t)(c + kk) * (uint32_t)r + (uint32_t)(r0 + 8 * v)) * 2u : kOOB;
            av[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0));
        }
    };
    auto store_a = [&](lds_char *dst, const uint4 (&av)[NAV]) {
#pragma unroll
        for (int j = 0; j < NAV; ++j) *(uint4 *)(dst + (lane + 64 * j) * 16) = av[j];
    };
    auto copy_a_generic = [&](int c, lds_char *dst) {
        for (int q = lane; q < F1S_UNIT * RL; q += 64) {
            const int kk = q / RL, rr = q % RL;
            uint16_t v = 0;
            if (c + kk < ke && r0 + rr < r) v = ad.A[(size_t)(c + kk) * r + r0 + rr];
            *(uint16_t *)(dst + q * 2) = v;
        }
    };

    // The loads of unit u+1 (A first, then X) are issued at the top of unit
    // u; storing A(u+1) to LDS at the end of the unit waits for A only, so
    // X(u+1) can still be in flight.  Units go in pairs so the two X register
    // sets alternate roles without copies (a copy would wait for its loads);
    // an odd count gets one extra unit, which reads and adds zeros.
    uint4 xr0[4], xr1[4], an[NAV];
    if (nu > 0) {
        load_x(kb, xr0);
        if (avec) {
            load_a(kb, an);
            store_a(slab0, an);
        } else {
            copy_a_generic(kb, slab0);
        }
    }
    auto unit = [&](int u, const uint4 (&xc)[4], uint4 (&xf)[4]) {
        const int c = kb + u * F1S_UNIT;
        // next unit's loads (past the range they read zeros)
        if (avec) load_a(c + F1S_UNIT, an);
        load_x(c + F1S_UNIT, xf);
        const lds_char *sl = slab0 + (u % NSLAB) * SLAB;
        uint32_t kw = 0;  // byte t: this lane's keep bits of step t
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c0 = c + 32 * t + 8 * g;
            uint4 xm = xc[t];
            uint32_t byte = 0xFFu;
            if (T != 0) {
                const PhiloxOut o = philox10(blk0 + (uint64_t)((c + 32 * t) >> 3), P.seed);
                byte = keep_and_mask(o, tm1x2, xc[t], xm);
            }
            kw |= (c0 < ke ? byte : 0u) << (8 * t);  // bits past k stay zero
            // rank-side fragment: k rows 32t + 8g + (0..7), rank 16 bt + l16
            const int kr = 32 * t + 8 * g + (l16 >> 2);
#pragma unroll
            for (int bt = 0; bt < MAXT; ++bt) {
                const lds_char *pa = sl + kr * (2 * RL) + (16 * bt + 4 * (l16 & 3)) * 2;
                const uint2 lo = lds_read_tr4(pa), hi = lds_read_tr4(pa + 4 * (2 * RL));
                acc[bt] = mfma16x16x32(xm, make_uint4(lo.x, lo.y, hi.x, hi.y), acc[bt]);
            }
        }
        if (P.keep_bits != nullptr && r0 == 0) {
            // 4x4 byte transpose across the lanes of a row (groups g): byte t of
            // lane g holds group g's bits of step t; afterwards lane g holds the
            // word of step g, byte j from group j.
            const uint32_t p1 = (uint32_t)__shfl_xor((int)kw, 16);
            kw = (g & 1) ? ((kw & 0xFF00FF00u) | ((p1 & 0xFF00FF00u) >> 8))
                         : ((kw & 0x00FF00FFu) | ((p1 & 0x00FF00FFu) << 8));
            const uint32_t p2 = (uint32_t)__shfl_xor((int)kw, 32);
            kw = (g & 2) ? ((kw & 0xFFFF0000u) | (p2 >> 16)) : ((kw & 0x0000FFFFu) | (p2 << 16));
            if (rvalid && c + 32 * g < ke) P.keep_bits[(size_t)row * P.KW + ((c >> 5) + g)] = kw;
        }
        lds_char *nx = slab0 + ((u + 1) % NSLAB) * SLAB;
        if (avec) store_a(nx, an);
        else copy_a_generic(c + F1S_UNIT, nx);
    };
    for (int u = 0; u < nu; u += 2) {
        unit(u, xr0, xr1);
        unit(u + 1, xr1, xr0);
    }

    // fixed-order sum of the waves' partial S (rows 4g+v, rank 16bt + l16);
    // the reduction buffer reuses the slabs once every wave is done with them
    __syncthreads();
    float *red = (float *)smem;  // [wave][16 rows][RL]
#pragma unroll
    for (int bt = 0; bt < MAXT; ++bt)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[(wave * 16 + 4 * g + v) * RL + 16 * bt + l16] = acc[bt][v];
    __syncthreads();
    for (int i = tid; i < 16 * RL; i += 64 * F1S_WAVES) {
        const int rr = i / RL, cl = i % RL;
        const int orow = row_lo + rr;
        if (orow >= row_hi) continue;
        float v = 0.f;
        if (r0 + cl < r) {
#pragma unroll
            for (int w = 0; w < F1S_WAVES; ++w) v += red[(w * 16 + rr) * RL + cl];
            v *= s;
        }
        if (cl < ncol) P.out[(size_t)orow * P.RS + r0 + cl] = v;
        // hi / lo columns run to s2_rp, past the S columns (ncol) of the last
        // rank tile: those past r are written as zeros too, since the forward
        // GEMM reads every one of them
        if (P.s2 != nullptr && r0 + cl < P.s2_rp) {
            // the forward epilogue's split of alpha*S, same arithmetic
            uint32_t hi, lo;
            split_bf16(ad.alpha * v, hi, lo);
            uint16_t *q = P.s2 + (size_t)orow * (2 * P.s2_rp) + r0 + cl;
            q[0] = (uint16_t)hi;
            q[P.s2_rp] = (uint16_t)lo;
        }
    }
}

// ----- F1 for ranks 33..128: one pass over X, A shared by 64 rows.
// Work-group = a 64-row chunk of one adapter (4 waves x 16 rows) x one slice
// of k.  Each 64-column unit of the slice -- the 64 rows of X (8 KiB) and A's
// 64 k-rows (64 x RP bf16) -- comes through a 3-stage ring of direct-to-LDS
// loads, so A is read once per 64 rows and every wave uses it (the small
// unit keeps two or three work-groups on a CU).
// Per 32-column step a lane hashes one Philox block for its row, masks its 8
// elements, and runs one MFMA per 16-rank block the chunk's adapter needs
// (the step is instantiated for 1, 2, 4 or 8 blocks).  The mask words are
// assembled across the lanes of a row (4 x 4 byte transpose) and stored by
// the slice that hashed them.  With one slice S (and the forward GEMM's hi |
// lo split of alpha*S) leaves the kernel; with several, each writes its
// partial and f1_reduce_kernel adds them in slice order.
struct F1WParams {
    const uint16_t *X;
    int m, k;
    RowWork work;  // 64-row chunks
    uint64_t seed, offset;
    uint32_t *keep_bits;
    int KW;
    float *S;
    int RS;
    float *part;  // several slices: [KS][m][RP], S before the dropout scale
    int ksl, KS;
    uint16_t *s2;  // one slice only (else f1_reduce_kernel writes it)
    int s2_rp;
};

template <int MAXT>
struct F1W {
    static constexpr int RP = 16 * MAXT;
    static constexpr int UNIT = 64;                 // k columns per stage (two MFMA steps)
    static constexpr int X_BYTES = 64 * UNIT * 2;   // 64 rows
    static constexpr int LDS = 3 * (X_BYTES + UNIT * RP * 2);  // 2 work-groups per CU at RP = 128, 3 below
};

// The ring of a chunk whose adapter needs NB 16-rank blocks: a stage holds X
// and A's 64 k-rows of 16 NB ranks (at least 2 KiB), and the ring takes as
// many stages (at most 8) as the launch's LDS holds -- chunks of small rank
// keep more of X in flight.  A loads: 1 KiB each, NB / 2 per wave (NB = 1:
// waves 0 and 1 one each).
template <int MAXT, int NB>
struct F1WRing {
    static constexpr int RPN = 16 * NB;
    static constexpr int A_BYTES = F1W<MAXT>::UNIT * RPN * 2;
    static constexpr int STAGE = F1W<MAXT>::X_BYTES + A_BYTES;
    static constexpr int NST = F1W<MAXT>::LDS / STAGE < 8 ? F1W<MAXT>::LDS / STAGE : 8;
    static constexpr int NAL = A_BYTES / 4096;      // A loads per wave per stage (NB >= 2)
    static constexpr int NPS_LO = 2 + NAL;          // loads per wave per stage, waves 2 and 3
    static constexpr int NPS_HI = NB == 1 ? 3 : NPS_LO;  // waves 0 and 1
};

// 32-byte chunk swizzle of A's slab rows (2*RP bytes): the 4 k-rows of a
// transposing read, and those 8 k-rows further on, land on distinct chunks.
template <int RP>
__device__ __forceinline__ int f1w_swz(int kr) {
    return ((kr & 3) | (((kr >> 3) & 1) << 2)) & (RP / 16 - 1);
}

template <int MAXT>
__global__ __launch_bounds__(256) void f1w_kernel(F1WParams P) {
    using C = F1W<MAXT>;
    constexpr int RP = C::RP;
    extern __shared__ uint4 f1w_smem[];
    lds_char *smem = (lds_char *)f1w_smem;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;

    int row_lo, row_hi;
    AdapterView ad;
    if (!resolve_chunk(P.work, blockIdx.x, P.m, row_lo, row_hi, ad)) return;
    const int r = ad.r;
    const int nbt = (r + 15) >> 4;
    const int ks = blockIdx.y, kb = ks * P.ksl, ke = min(P.k, kb + P.ksl);
    if (kb >= ke) return;
    const int nu = (ke - kb + C::UNIT - 1) / C::UNIT;
    const int nrows = row_hi - row_lo;
    const uint32_t T = drop_threshold(ad.p);
    const uint32_t tm1x2 = ((T - 1u) & 0xFFFFu) * 0x00010001u;  // used only when T >= 1
    const float s = drop_scale(ad.p);
    auto clampb = [](uint64_t v) { return (uint32_t)(v < 0x7FFFFFF0ull ? v : 0x7FFFFFF0ull); };
    const sgpr4_t dX = make_desc(P.X + (size_t)row_lo * P.k, clampb((uint64_t)nrows * P.k * 2));
    const bool avec = (r & 7) == 0 && (((uintptr_t)ad.A) & 15) == 0;
    const uint64_t abytes = (uint64_t)P.k * r * 2;
    const sgpr4_t dA = make_desc(ad.A, clampb(abytes));

    // X: load j of wave w covers rows 16w + 8j + lane/8, 16-byte chunk
    // position lane%8 of the 128-byte LDS row, which holds logical chunk
    // (lane%8) ^ (row/2 % 8) (16 consecutive rows read at one logical chunk
    // hit 16 distinct bank groups)
    constexpr int UNIT = C::UNIT;
    uint32_t offX[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        offX[j] = (16 * wave + row < nrows) ? (uint32_t)(((size_t)(16 * wave + row) * P.k + 8 * c) * 2) : kOOBL;
    }
    const int row = row_lo + 16 * wave + l16;
    const bool rvalid = 16 * wave + l16 < nrows;
    // Philox block of the lane's first element in a step at column c: (offset
    // + row*k + c + 8g) / 8, every term a multiple of 8
    const uint64_t blk0 = (P.offset >> 3) + (uint64_t)(rvalid ? row : row_lo) * (uint64_t)(P.k >> 3) + (uint64_t)g;

    auto body = [&](auto nb_c) {
        constexpr int NB = decltype(nb_c)::value;
        using R = F1WRing<MAXT, NB>;
        constexpr int RPN = R::RPN;
        constexpr int NST = R::NST;
        auto issue = [&](int u, int st) {
            const uint32_t base = lds0 + st * R::STAGE;
            const int c0 = kb + UNIT * u;
            const bool live = u < nu;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int row = 8 * j + (lane >> 3);
                const int c = (lane & 7) ^ ((row >> 1) & 7);
                const bool ok = live && offX[j] != kOOBL && c0 + 8 * c < ke;
                dma16(dX, ok ? offX[j] + (uint32_t)c0 * 2u : kOOBL, base + wave * 2048 + j * 1024);
            }
            const uint32_t abase = base + C::X_BYTES;
            if (avec) {
                auto a_load = [&](int q) {
                    const int pos = q * 1024 + lane * 16;
                    const int kr = pos / (2 * RPN), within = pos % (2 * RPN);
                    const int cl = (within >> 5) ^ f1w_swz<RPN>(kr), h = (within >> 4) & 1;
                    const int rank = 16 * cl + 8 * h;
                    const bool ok = live && c0 + kr < ke && rank < r;
                    dma16(dA, ok ? (uint32_t)(((size_t)(c0 + kr) * r + rank) * 2) : kOOBL, abase + q * 1024);
                };
                if constexpr (NB == 1) {
                    if (wave < 2) a_load(wave);
                } else {
#pragma unroll
                    for (int i = 0; i < R::NAL; ++i) a_load(wave * R::NAL + i);
                }
            } else {
                // A neither 16-byte aligned nor of a rank divisible by 8: element copy
                lds_char *dst = smem + st * R::STAGE + C::X_BYTES;
                for (int idx = tid; idx < UNIT * RPN; idx += 256) {
                    const int kr = idx / RPN, rank = idx % RPN;
                    uint16_t v = 0;
                    if (live && c0 + kr < ke && rank < r) v = ad.A[(size_t)(c0 + kr) * r + rank];
                    *(uint16_t *)(dst + kr * (2 * RPN) + (((rank >> 4) ^ f1w_swz<RPN>(kr)) << 5) + (rank & 15) * 2) = v;
                }
            }
        };
        // stage u+1 landed: every load but those of the NST-2 stages issued after it
        auto wait_ring = [&]() {
            if constexpr (R::NPS_HI != R::NPS_LO) {
                if (wave < 2) wait_vmcnt<R::NPS_HI * (NST - 2)>();
                else wait_vmcnt<R::NPS_LO * (NST - 2)>();
            } else {
                wait_vmcnt<R::NPS_LO * (NST - 2)>();
            }
        };
        f32x4_t acc[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < NST - 1; ++q) issue(q, q);
        wait_ring();
        __syncthreads();
        int st = 0, ls = NST - 1;
        uint32_t kw = 0;  // byte t: this lane's keep bits of step t of the 128-column pair of units
        for (int u = 0; u < nu; ++u) {
            issue(u + NST - 1, ls);
            const lds_char *xt = smem + st * R::STAGE + wave * 2048;
            const lds_char *at = smem + st * R::STAGE + C::X_BYTES;
            const int c = kb + UNIT * u;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint4 x = *(const uint4 *)(xt + l16 * 128 + (((4 * t + g) ^ ((l16 >> 1) & 7)) << 4));
                uint4 xm = x;
                uint32_t byte = 0xFFu;
                if (T != 0) {
                    const PhiloxOut o = philox10(blk0 + (uint64_t)((c + 32 * t) >> 3), P.seed);
                    byte = keep_and_mask(o, tm1x2, x, xm);
                }
                kw |= (c + 32 * t + 8 * g < ke ? byte : 0u) << (8 * (2 * (u & 1) + t));  // bits past the slice stay zero
                const int kr = 32 * t + 8 * g + (l16 >> 2);
                const int sw = f1w_swz<RPN>(kr);
#pragma unroll
                for (int bt = 0; bt < NB; ++bt) {
                    const lds_char *pa = at + kr * (2 * RPN) + ((bt ^ sw) << 5) + 8 * (l16 & 3);
                    const uint2 lo = lds_read_tr4(pa), hi = lds_read_tr4(pa + 4 * (2 * RPN));
                    acc[bt] = mfma16x16x32(xm, make_uint4(lo.x, lo.y, hi.x, hi.y), acc[bt]);
                }
            }
            if (P.keep_bits != nullptr && ((u & 1) || u == nu - 1)) {
                const int c = kb + UNIT * (u & ~1);  // first column of the pair
                // 4x4 byte transpose across the lanes of a row (groups g):
                // afterwards lane g holds the word of step g, byte j from group j
                const uint32_t p1 = (uint32_t)__shfl_xor((int)kw, 16);
                kw = (g & 1) ? ((kw & 0xFF00FF00u) | ((p1 & 0xFF00FF00u) >> 8))
                             : ((kw & 0x00FF00FFu) | ((p1 & 0x00FF00FFu) << 8));
                const uint32_t p2 = (uint32_t)__shfl_xor((int)kw, 32);
                kw = (g & 2) ? ((kw & 0xFFFF0000u) | (p2 >> 16)) : ((kw & 0x0000FFFFu) | (p2 << 16));
                if (rvalid && c + 32 * g < ke) P.keep_bits[(size_t)row * P.KW + ((c >> 5) + g)] = kw;
                kw = 0;
            }
            wait_ring();
            __syncthreads();
            st = st == NST - 1 ? 0 : st + 1;
            ls = ls == NST - 1 ? 0 : ls + 1;
        }
        wait_vmcnt<0>();
        // rows 4g + v of the wave, rank 16 bt + l16
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int lr = 16 * wave + 4 * g + v;
            if (lr >= nrows) continue;
            const int orow = row_lo + lr;
            if (P.KS == 1) {
                for (int rr = l16; rr < P.RS; rr += 16) {
                    float val = 0.f;
#pragma unroll
                    for (int bt = 0; bt < NB; ++bt)
                        if (rr == 16 * bt + l16 && rr < r) val = acc[bt][v] * s;
                    P.S[(size_t)orow * P.RS + rr] = val;
                }
                if (P.s2 != nullptr) {
                    for (int rr = l16; rr < P.s2_rp; rr += 16) {
                        float val = 0.f;
#pragma unroll
                        for (int bt = 0; bt < NB; ++bt)
                            if (rr == 16 * bt + l16 && rr < r) val = acc[bt][v] * s;
                        uint32_t hi, lo;
                        split_bf16(ad.alpha * val, hi, lo);
                        uint16_t *q = P.s2 + (size_t)orow * (2 * P.s2_rp) + rr;
                        q[0] = (uint16_t)hi;
                        q[P.s2_rp] = (uint16_t)lo;
                    }
                }
            } else {
                float *pp = P.part + ((size_t)ks * P.m + orow) * RP;
#pragma unroll
                for (int bt = 0; bt < MAXT; ++bt) {
                    float val = 0.f;
#pragma unroll
                    for (int b2 = 0; b2 < NB; ++b2)
                        if (b2 == bt) val = acc[b2][v];
                    pp[16 * bt + l16] = val;
                }
            }
        }
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    using I8 = std::integral_constant<int, 8>;
    if constexpr (MAXT == 4) {
        if (nbt <= 1) body(I1{});
        else if (nbt <= 2) body(I2{});
        else body(I4{});
    } else {
        if (nbt <= 1) body(I1{});
        else if (nbt <= 2) body(I2{});
        else if (nbt <= 4) body(I4{});
        else body(I8{});
    }
}

// S (and the forward GEMM's split of alpha*S) from f1w_kernel's slice
// partials, added in slice order; one work-group per 64-row chunk.
__global__ __launch_bounds__(256) void f1_reduce_kernel(F1WParams P, int RP) {
    int row_lo, row_hi;
    AdapterView ad;
    if (!resolve_chunk(P.work, blockIdx.x, P.m, row_lo, row_hi, ad)) return;
    const int r = ad.r;
    const float s = drop_scale(ad.p);
    const int nrows = row_hi - row_lo;
    const int width = max(P.RS, P.s2 != nullptr ? P.s2_rp : 0);
    const int e = blockIdx.y * 256 + threadIdx.x;  // one output element per thread
    if (e >= nrows * width) return;
    const int lr = e / width, rr = e - lr * width;
    const int orow = row_lo + lr;
    float v = 0.f;
    if (rr < r) {
        const float *src = P.part + (size_t)orow * RP + rr;
        const size_t qs = (size_t)P.m * RP;
        int q = 0;
        for (; q + 4 <= P.KS; q += 4) {
            const float a0 = src[q * qs], a1 = src[(q + 1) * qs], a2 = src[(q + 2) * qs], a3 = src[(q + 3) * qs];
            v = (((v + a0) + a1) + a2) + a3;
        }
        for (; q < P.KS; ++q) v += src[q * qs];
        v *= s;
    }
    if (rr < P.RS) P.S[(size_t)orow * P.RS + rr] = v;
    if (P.s2 != nullptr && rr < P.s2_rp) {
        uint32_t hi, lo;
        split_bf16(ad.alpha * v, hi, lo);
        uint16_t *q2 = P.s2 + (size_t)orow * (2 * P.s2_rp) + rr;
        q2[0] = (uint16_t)hi;
        q2[P.s2_rp] = (uint16_t)lo;
    }
}

// ===========================================================================
// Fixed-order sum of split partials: out[i] = sum_p part[p*stride + i].  A
// work-group covers 64 float4 columns; its four waves each sum every fourth
// part, and the four partial sums are added in a fixed order (bitwise
// reproducible).
// ===========================================================================
__device__ __forceinline__ void sum_partials_block(const float *part, int nparts, size_t stride, size_t count,
                                                   float *out, int block) {
    __shared__ float4 red[4][64];
    const int t = threadIdx.x, pg = t >> 6, c = t & 63;
    const size_t i4 = ((size_t)block * 64 + c) * 4;
    const bool vec = (stride & 3) == 0 && (((uintptr_t)part) & 15) == 0;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i4 < count) {
        if (vec && i4 + 4 <= count) {
#pragma unroll 4
            for (int p = pg; p < nparts; p += 4) {
                const float4 b = *(const float4 *)(part + (size_t)p * stride + i4);
                a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
            }
        } else {
            float v[4] = {0.f, 0.f, 0.f, 0.f};
            for (int p = pg; p < nparts; p += 4)
                for (int e = 0; e < 4; ++e)
                    if (i4 + e < count) v[e] += part[(size_t)p * stride + i4 + e];
            a = make_float4(v[0], v[1], v[2], v[3]);
        }
    }
    red[pg][c] = a;
    __syncthreads();
    if (pg == 0 && i4 < count) {
        float4 r0 = red[0][c];
#pragma unroll
        for (int q = 1; q < 4; ++q) {
            const float4 b = red[q][c];
            r0.x += b.x; r0.y += b.y; r0.z += b.z; r0.w += b.w;
        }
        const float rv[4] = {r0.x, r0.y, r0.z, r0.w};
        for (int e = 0; e < 4; ++e)
            if (i4 + e < count) out[i4 + e] = rv[e];
    }
}

__global__ __launch_bounds__(256) void sum_partials_kernel(const float *part, int nparts, size_t stride,
                                                           size_t count, float *out) {
    sum_partials_block(part, nparts, stride, count, out, blockIdx.x);
}

// ===========================================================================
// B1: dS and dB from one pass over dY (juhe.plus blog, section 4.1, backward
// item 3: fuse the dS and dB computations so dY is loaded once).
// Work-group = one chunk (<= 256 rows) x C1 columns, in 64-row sub-blocks.
//   dS part: wave w owns 16 rows; A-frag = dY row (LDS Ys), B-frag = B row
//            (LDS Bs), K = the C1 columns -> partial over this column tile.
//   dB part: wave w owns C1/4 columns; A-frag = (alpha*S)^T (LDS Sts, fp32 ->
//            hi/lo), B-frag = dY column (8 rows gathered from Ys), K = rows.
// ===========================================================================
struct B1Params {
    const uint16_t *dY;
    const float *S;
    int m, n, RS;
    RowWork work;
    float *dSpart;  // [CT][m][RS]
    float *dBpart;  // [chunk][RS][n]
    int r_lds;
    int tiled;  // rank tiles of 32 (blockIdx.z); S staged 32 columns per row (RS % 4 == 0)
};

template <int C1, int MAXT>
__global__ __launch_bounds__(256) void b1_kernel(B1Params P) {
    constexpr int LDY = C1 + 8;    // Ys / Bs row stride (elements)
    constexpr int LDS_S = 64 + 4;  // Sts row stride (floats)
    constexpr int NBW = C1 / 64;   // 16-wide column blocks per wave (dB part)
    extern __shared__ uint4 b1_smem[];
    uint16_t *Bs = (uint16_t *)b1_smem;               // [r_lds][LDY]
    uint16_t *Ys = Bs + (size_t)P.r_lds * LDY;        // [64][LDY]
    float *Sts = (float *)(Ys + 64 * LDY);            // [r_lds][LDS_S]

    int row_lo, row_hi;
    AdapterView ad;
    if (!resolve_chunk(P.work, blockIdx.x, P.m, row_lo, row_hi, ad)) return;
    const int r = ad.r;
    const int nbt = (r + 15) >> 4;
    const int rpad = nbt * 16;
    const float alpha = ad.alpha;
    const int ct = blockIdx.y;
    const int n0 = ct * C1;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, li = lane & 15;

    for (int idx = tid; idx < rpad * C1; idx += 256) {
        const int rr = idx / C1, j = idx - rr * C1;
        uint16_t v = 0;
        if (rr < r && n0 + j < P.n) v = ad.B[(size_t)rr * P.n + n0 + j];
        Bs[rr * LDY + j] = v;
    }

    f32x4_t accB[MAXT][NBW];
#pragma unroll
    for (int a = 0; a < MAXT; ++a)
#pragma unroll
        for (int b = 0; b < NBW; ++b) accB[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Register staging of one 64-row sub-block: dY (64 x C1) and alpha*S (64 x rpad).
    constexpr int NLY = C1 / 32;      // 16-byte dY loads per thread
    constexpr int NLS = MAXT * 4;     // S values per thread (64 * 16*MAXT / 256)
    uint4 yv[NLY];
    float sv[NLS];
    auto load_sub = [&](int rs) {
#pragma unroll
        for (int j = 0; j < NLY; ++j) {
            const int v = tid + 256 * j;
            const int rrow = v / (C1 / 8), cv = v - rrow * (C1 / 8);
            const int row = rs + rrow, col = n0 + cv * 8;
            yv[j] = (row < row_hi && col < P.n) ? *(const uint4 *)(P.dY + (size_t)row * P.n + col)
                                                : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < NLS; ++j) {
            const int idx = tid + 256 * j;
            const int rrow = idx / rpad, rr = idx - rrow * rpad;
            const int row = rs + rrow;
            sv[j] = (idx < 64 * rpad && row < row_hi && rr < r) ? alpha * P.S[(size_t)row * P.RS + rr] : 0.f;
        }
    };
    load_sub(row_lo);
    for (int rs = row_lo; rs < row_hi; rs += 64) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NLY; ++j) {
            const int v = tid + 256 * j;
            const int rrow = v / (C1 / 8), cv = v - rrow * (C1 / 8);
            *(uint4 *)&Ys[rrow * LDY + cv * 8] = yv[j];
        }
#pragma unroll
        for (int j = 0; j < NLS; ++j) {
            const int idx = tid + 256 * j;
            if (idx < 64 * rpad) {
                const int rrow = idx / rpad, rr = idx - rrow * rpad;
                Sts[rr * LDS_S + rrow] = sv[j];
            }
        }
        __syncthreads();
        if (rs + 64 < row_hi) load_sub(rs + 64);  // in flight during the MFMA work below

        // ---- dS partial for rows rs + 16*wave .. +16 over this column tile
        {
            f32x4_t accS[MAXT];
#pragma unroll
            for (int t = 0; t < MAXT; ++t) accS[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
            for (int t = 0; t < C1 / 32; ++t) {
                const uint4 af = *(const uint4 *)&Ys[(wave * 16 + li) * LDY + 32 * t + 8 * g];
#pragma unroll
                for (int bt = 0; bt < MAXT; ++bt) {
                    if (bt < nbt) {
                        const uint4 bf = *(const uint4 *)&Bs[(bt * 16 + li) * LDY + 32 * t + 8 * g];
                        accS[bt] = mfma16x16x32(af, bf, accS[bt]);
                    }
                }
            }
            float *dsp = P.dSpart + (size_t)ct * P.m * P.RS;
#pragma unroll
            for (int bt = 0; bt < MAXT; ++bt) {
                if (bt < nbt) {
                    const int col = bt * 16 + li;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int orow = rs + wave * 16 + 4 * g + v;
                        if (orow < row_hi && col < P.RS)
                            dsp[(size_t)orow * P.RS + col] = col < r ? alpha * accS[bt][v] : 0.f;
                    }
                }
            }
            for (int col = rpad + li; col < P.RS; col += 16) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int orow = rs + wave * 16 + 4 * g + v;
                    if (orow < row_hi) dsp[(size_t)orow * P.RS + col] = 0.f;
                }
            }
        }

        // ---- dB partial: columns wave*C1/4 .., K = the 64 rows
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            uint4 bfr[NBW];
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int col = (wave * NBW + nb) * 16 + li;
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = Ys[(32 * t + 8 * g + e) * LDY + col];
                bfr[nb] = make_uint4(pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7]));
            }
#pragma unroll
            for (int bt = 0; bt < MAXT; ++bt) {
                if (bt < nbt) {
                    const float4 s0 = *(const float4 *)&Sts[(bt * 16 + li) * LDS_S + 32 * t + 8 * g];
                    const float4 s1 = *(const float4 *)&Sts[(bt * 16 + li) * LDS_S + 32 * t + 8 * g + 4];
                    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
                    uint4 ahi, alo;
                    split_frag(sv, ahi, alo);
#pragma unroll
                    for (int nb = 0; nb < NBW; ++nb) {
                        accB[bt][nb] = mfma16x16x32(ahi, bfr[nb], accB[bt][nb]);
                        accB[bt][nb] = mfma16x16x32(alo, bfr[nb], accB[bt][nb]);
                    }
                }
            }
        }
    }

    float *dbp = P.dBpart + (size_t)blockIdx.x * P.RS * P.n;
#pragma unroll
    for (int bt = 0; bt < MAXT; ++bt) {
        if (bt < nbt) {
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int col = n0 + (wave * NBW + nb) * 16 + li;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int rr = bt * 16 + 4 * g + v;
                    if (rr < r && col < P.n) dbp[(size_t)rr * P.n + col] = accB[bt][nb][v];
                }
            }
        }
    }
}

// ===========================================================================
// B2: dA = s*(keep.X)^T dS (the backward's dA step; the pages number the
// backward kernels 3 and 5 and leave 4 out -- dA is taken as that step).
// Work-group = one chunk (<= 256 rows) x C2 columns of k, in 64-row
// sub-blocks.  Each thread loads an 8x8 block of X (8 rows x 16 B), applies
// the stored mask, transposes it in registers and writes Xt[kk][row] so the
// MFMA A-fragments (8 consecutive rows of one column) are 16-B LDS reads.
// ===========================================================================
struct B2Params {
    const uint16_t *X;
    const uint32_t *keep;
    const float *dS;
    int m, k, RS, KW;
    RowWork work;
    float *dApart;  // [chunk][k][RS]
    int r_lds;
    int tiled;  // rank tiles of 32 (blockIdx.z); dS staged 32 columns per row (RS % 4 == 0)
};

template <int C2, int MAXT>
__global__ __launch_bounds__(256) void b2_kernel(B2Params P) {
    constexpr int LDX = 64 + 8;      // Xt row stride (elements)
    constexpr int LDS_S = 64 + 4;    // dSts row stride (floats)
    constexpr int MBW = C2 / 64;     // 16-wide k blocks per wave
    extern __shared__ uint4 b2_smem[];
    uint16_t *Xt = (uint16_t *)b2_smem;            // [C2][LDX]
    float *dSts = (float *)(Xt + (size_t)C2 * LDX);  // [r_lds][LDS_S]

    int row_lo, row_hi;
    AdapterView ad;
    if (!resolve_chunk(P.work, blockIdx.x, P.m, row_lo, row_hi, ad)) return;
    const int r = ad.r;
    const int nbt = (r + 15) >> 4;
    const int rpad = nbt * 16;
    const float s = drop_scale(ad.p);
    const int k0 = blockIdx.y * C2;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, li = lane & 15;

    f32x4_t accA[MBW][MAXT];
#pragma unroll
    for (int a = 0; a < MBW; ++a)
#pragma unroll
        for (int b = 0; b < MAXT; ++b) accA[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Register staging of one 64-row sub-block: an 8x8 block of X with its
    // keep bytes per thread (C2 == 256: every thread; 128: half) and s*dS.
    constexpr int NBLK = (8 * (C2 / 8) + 255) / 256;  // 8x8 blocks per thread
    constexpr int NLS = MAXT * 4;
    uint4 xv[NBLK][8];
    uint32_t kb8[NBLK][8];
    float dv[NLS];
    auto load_sub = [&](int rs) {
#pragma unroll
        for (int q = 0; q < NBLK; ++q) {
            const int blk = tid + 256 * q;
            const int rb = blk / (C2 / 8), cb = blk - rb * (C2 / 8);
            const int col = k0 + cb * 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int row = rs + rb * 8 + e;
                const bool ok = blk < 8 * (C2 / 8) && row < row_hi && col < P.k;
                xv[q][e] = ok ? *(const uint4 *)(P.X + (size_t)row * P.k + col) : make_uint4(0, 0, 0, 0);
                kb8[q][e] = (ok && P.keep != nullptr) ? P.keep[(size_t)row * P.KW + (col >> 5)] >> (col & 31) : 0xFFu;
            }
        }
#pragma unroll
        for (int j = 0; j < NLS; ++j) {
            const int idx = tid + 256 * j;
            const int rrow = idx / rpad, rr = idx - rrow * rpad;
            const int row = rs + rrow;
            dv[j] = (idx < 64 * rpad && row < row_hi && rr < r) ? s * P.dS[(size_t)row * P.RS + rr] : 0.f;
        }
    };
    load_sub(row_lo);
    for (int rs = row_lo; rs < row_hi; rs += 64) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NBLK; ++q) {
            const int blk = tid + 256 * q;
            if (blk < 8 * (C2 / 8)) {
                const int rb = blk / (C2 / 8), cb = blk - rb * (C2 / 8);
                uint4 v[8], o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = apply_keep(xv[q][e], kb8[q][e] & 0xFFu);
                transpose8x8(v, o);
#pragma unroll
                for (int c = 0; c < 8; ++c) *(uint4 *)&Xt[(cb * 8 + c) * LDX + rb * 8] = o[c];
            }
        }
#pragma unroll
        for (int j = 0; j < NLS; ++j) {
            const int idx = tid + 256 * j;
            if (idx < 64 * rpad) {
                const int rrow = idx / rpad, rr = idx - rrow * rpad;
                dSts[rr * LDS_S + rrow] = dv[j];
            }
        }
        __syncthreads();
        if (rs + 64 < row_hi) load_sub(rs + 64);  // in flight during the MFMA work below

#pragma unroll
        for (int t = 0; t < 2; ++t) {
            uint4 af[MBW];
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
                af[mb] = *(const uint4 *)&Xt[((wave * MBW + mb) * 16 + li) * LDX + 32 * t + 8 * g];
#pragma unroll
            for (int bt = 0; bt < MAXT; ++bt) {
                if (bt < nbt) {
                    const float4 s0 = *(const float4 *)&dSts[(bt * 16 + li) * LDS_S + 32 * t + 8 * g];
                    const float4 s1 = *(const float4 *)&dSts[(bt * 16 + li) * LDS_S + 32 * t + 8 * g + 4];
                    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
                    uint4 bhi, blo;
                    split_frag(sv, bhi, blo);
#pragma unroll
                    for (int mb = 0; mb < MBW; ++mb) {
                        accA[mb][bt] = mfma16x16x32(af[mb], bhi, accA[mb][bt]);
                        accA[mb][bt] = mfma16x16x32(af[mb], blo, accA[mb][bt]);
                    }
                }
            }
        }
    }

    float *dap = P.dApart + (size_t)blockIdx.x * P.k * P.RS;
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
#pragma unroll
        for (int bt = 0; bt < MAXT; ++bt) {
            if (bt < nbt) {
                const int rr = bt * 16 + li;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int kk = k0 + (wave * MBW + mb) * 16 + 4 * g + v;
                    if (kk < P.k && rr < r) dap[(size_t)kk * P.RS + rr] = accA[mb][bt][v];
                }
            }
        }
    }
}

// ===========================================================================
// Streaming variants of B1 and B2 for ranks <= 32 per launch slice (ranks up to
// 128 in rank tiles of 32, grid dimension z).  The full-size operand
// (dY or X) and the small per-row operands (alpha*S or dS, the keep words)
// flow global -> LDS through a 3-stage ring of direct-to-LDS loads, so two
// sub-blocks are in flight while a third is consumed and no VGPRs stage data.
// The tiles use the 512-byte-row swizzle and transposing reads of
// device_common.hpp (swz512_off, tile_rows8).
// ===========================================================================

// ----- B2 streaming: sub-blocks of 32 rows; stage = X 16 KiB + 8 aux KiB
constexpr int B2S_ROWS = 32, B2S_X = 32 * 512, B2S_STAGE = B2S_X + 8 * 1024, B2S_NST = 3;

template <int MAXT>
__global__ __launch_bounds__(256) void b2s_kernel(B2Params P) {
    extern __shared__ uint4 b2s_smem[];
    lds_char *smem = (lds_char *)b2s_smem;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    int row_lo, row_hi;
    AdapterView ad;
    if (!resolve_chunk(P.work, blockIdx.x, P.m, row_lo, row_hi, ad)) return;
    const int r = ad.r;
    constexpr int RL = 16 * MAXT;
    // rank tile (tiled launches): ranks r0 .. r0+RL-1; dS rows staged as RL
    // floats (else the whole RS-float rows, r0 = 0)
    const int r0 = P.tiled ? (int)blockIdx.z * RL : 0;
    if (r0 >= r) return;  // partial columns past r are never read
    const int rt = min(r - r0, RL);
    const int nbt = (rt + 15) >> 4;
    const int sst = P.tiled ? 32 : P.RS;  // LDS row stride of the staged dS (tiled: RL = 32)
    const float s = drop_scale(ad.p);
    const int k0 = blockIdx.y * 256;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, li = lane & 15;
    const int nrows = row_hi - row_lo;
    const int nsb = (nrows + B2S_ROWS - 1) / B2S_ROWS;
    const bool has_mask = P.keep != nullptr;
    auto clampb = [](uint64_t v) { return (uint32_t)(v < 0x7FFFFFF0ull ? v : 0x7FFFFFF0ull); };
    const sgpr4_t dX = make_desc(P.X + (size_t)row_lo * P.k, clampb((uint64_t)nrows * P.k * 2));
    const sgpr4_t dK = make_desc(has_mask ? P.keep + (size_t)row_lo * P.KW : P.keep,
                                 has_mask ? clampb((uint64_t)nrows * P.KW * 4) : 0u);
    const sgpr4_t dD = make_desc(P.dS + (size_t)row_lo * P.RS, clampb((uint64_t)nrows * P.RS * 4));

    // this lane's DMA offsets inside sub-block 0 (X: 4 loads, aux: slots 2w, 2w+1)
    uint32_t offX[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int rr = 2 * (4 * wave + j) + (lane >> 5);
        const int col = k0 + 8 * ((lane & 31) ^ swz512(rr));
        offX[j] = col < P.k ? (uint32_t)(((size_t)rr * P.k + col) * 2) : kOOBL;
    }
    const uint32_t dsb = (uint32_t)(B2S_ROWS * P.RS * 4);  // dS bytes per sub-block
    auto issue = [&](int sb, int stage) {
        const uint32_t base = lds0 + stage * B2S_STAGE;
        const uint32_t xo = (uint32_t)((size_t)sb * B2S_ROWS * P.k * 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(dX, offX[j] == kOOBL ? kOOBL : offX[j] + xo, base + (4 * wave + j) * 1024);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int slot = 2 * wave + q;
            const uint32_t dst = base + B2S_X + slot * 1024;
            if (slot == 0) {
                const int w0 = (k0 >> 5) + 4 * (lane & 1);
                const uint32_t off = (has_mask && w0 < P.KW)
                    ? (uint32_t)((((size_t)sb * B2S_ROWS + (lane >> 1)) * P.KW + w0) * 4) : kOOBL;
                dma16(dK, off, dst);
            } else if (P.tiled) {
                // slot q: rows 8(q-1) + lane/8, 16-byte chunk lane % 8 of the tile's columns
                const int row = 8 * (slot - 1) + (lane >> 3), cc = r0 + 4 * (lane & 7);
                const uint32_t off = (slot <= 4 && cc < P.RS)
                    ? (uint32_t)((((size_t)sb * B2S_ROWS + row) * P.RS + cc) * 4) : kOOBL;
                dma16(dD, off, dst);
            } else {
                const uint32_t b = (uint32_t)(slot - 1) * 1024 + lane * 16;
                dma16(dD, b < dsb ? (uint32_t)sb * dsb + b : kOOBL, dst);
            }
        }
    };

    f32x4_t acc[4][MAXT];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < MAXT; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    issue(0, 0);
    issue(1, 1);
    wait_vmcnt<6>();
    __syncthreads();
    int stage = 0, lstage = 2;
    for (int sb = 0; sb < nsb; ++sb) {
        issue(sb + 2, lstage);
        const lds_char *xt = smem + stage * B2S_STAGE;
        const uint32_t *mk = (const uint32_t *)(xt + B2S_X);
        const float *ds = (const float *)(xt + B2S_X + 1024);
        // dS operand (N = rank): rows 8g..8g+7 of rank column 16*bt + li, times s
        uint4 bhi[MAXT], blo[MAXT];
#pragma unroll
        for (int bt = 0; bt < MAXT; ++bt) {
            float v[8];
            const int rr = 16 * bt + li;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // in-bounds for every lane (rows < 32, RS and rr < 32): read, then select
                const float dv = ds[(8 * g + e) * sst + rr];
                v[e] = (bt < nbt && rr < rt) ? s * dv : 0.f;
            }
            split_frag(v, bhi[bt], blo[bt]);
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int cb = 4 * wave + mb;  // 16-column block of this work-group's 256
            uint4 xf = tile_rows8(xt, 8 * g, cb, lane);
            if (has_mask) {
                const int bit = 16 * (cb & 1) + li;
                uint32_t m[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t w0 = mk[(8 * g + 2 * q) * 8 + (cb >> 1)];
                    const uint32_t w1 = mk[(8 * g + 2 * q + 1) * 8 + (cb >> 1)];
                    const uint32_t e0 = (uint32_t)__builtin_amdgcn_sbfe((int)w0, bit, 1);
                    const uint32_t e1 = (uint32_t)__builtin_amdgcn_sbfe((int)w1, bit, 1);
                    m[q] = (e0 & 0x0000FFFFu) | (e1 & 0xFFFF0000u);
                }
                xf = make_uint4(xf.x & m[0], xf.y & m[1], xf.z & m[2], xf.w & m[3]);
            }
#pragma unroll
            for (int bt = 0; bt < MAXT; ++bt) {
                if (bt < nbt) {
                    acc[mb][bt] = mfma16x16x32(xf, bhi[bt], acc[mb][bt]);
                    acc[mb][bt] = mfma16x16x32(xf, blo[bt], acc[mb][bt]);
                }
            }
        }
        wait_vmcnt<6>();
        __syncthreads();
        stage = stage == B2S_NST - 1 ? 0 : stage + 1;
        lstage = lstage == B2S_NST - 1 ? 0 : lstage + 1;
    }
    wait_vmcnt<0>();

    float *dap = P.dApart + (size_t)blockIdx.x * P.k * P.RS;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int bt = 0; bt < MAXT; ++bt) {
            if (bt < nbt) {
                const int rr = bt * 16 + li;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int kk = k0 + (4 * wave + mb) * 16 + 4 * g + v;
                    if (kk < P.k && rr < rt) dap[(size_t)kk * P.RS + r0 + rr] = acc[mb][bt][v];
                }
            }
        }
    }
}

// ----- B2, one pass over X for ranks up to 128.
// Work-group = one work item (rows of one adapter) x 256 columns of k, all
// ranks at once (16 * MAXT of them).  Rows go in sub-blocks of 32 through a
// 3- or 4-stage ring of direct-to-LDS loads: X (32 x 256 bf16, swizzled 512-byte
// rows), the rows' mask words (32 x 8 words) and the rank-side operand.
// Wave w owns the 16-column blocks 4w .. 4w+3 and accumulates
// (s*keep.X)^T dS for them over all the item's rows, then writes its part of
// the item's partial; dA_reduce_kernel adds the partials of each adapter.
// The rank-side operand is s*dS split into bf16 hi + lo, the same for all
// four waves.  Up to 32 ranks each wave splits the fp32 dS rows itself.
// Above that (MAXT >= 4) the split comes ready from B1's finishing launch
// (rows of [hi of RPa ranks | lo of RPa ranks], RPa the item's 16-rank
// blocks) and is loaded straight into a 32 x 512-byte tile with X's chunk
// swizzle, which the MFMAs read with transposing LDS reads: no split work
// and no extra barrier per sub-block.
struct B2WParams {
    const uint16_t *X;
    const uint32_t *keep;
    const float *dS;
    const uint16_t *dss;  // MAXT >= 4: split s*dS rows, dss_ld bf16 apart
    int dss_ld;
    int m, k, RS, KW;
    RowWork work;   // work items: the router's backward table, or rows_per_chunk rows
    int nct;        // column tiles of 256
    float *part;    // [item][nct][256][RPT]
};

template <int MAXT>
struct B2W {
    static constexpr int RPT = 16 * MAXT;                  // ranks per partial row
    static constexpr bool PRESPLIT = MAXT >= 4;            // rank side from the split rows
    static constexpr int X_BYTES = 32 * 512;
    // fp32 dS rows: aux 1 KiB loads of mask, then dS (slots past NA load zeros
    // into the stage's spare kibibytes); split rows: 4 loads per wave of the
    // 16 KiB tile, plus the mask (wave 0) or a dummy load (waves 1..3)
    static constexpr int NA = PRESPLIT ? 1 : 1 + (32 * RPT * 4) / 1024;
    static constexpr int NPW = PRESPLIT ? 5 : (NA + 3) / 4;  // aux loads per wave
    static constexpr int SPL_OFF = X_BYTES;                   // split tile (PRESPLIT)
    static constexpr int MASK_OFF = PRESPLIT ? X_BYTES + 16384 : X_BYTES;
    static constexpr int DS_OFF = X_BYTES + 1024;             // fp32 dS rows (not PRESPLIT)
    static constexpr int STAGE = PRESPLIT ? X_BYTES + 16384 + 2048 : X_BYTES + 4 * NPW * 1024;
    static constexpr int NST = MAXT == 2 ? 3 : 4;           // ring depth
    static constexpr int LDS = NST * STAGE;
};

// Word c (0..7) of row t (0..31) of a 32 x 32-byte mask tile whose 16-byte
// slots are permuted: row-half s = 2 t + c / 4 sits in slot s ^ (((t >> 3) & 3) << 2).
// Rows 8g + j of the four 16-lane groups g then fall in four different bank
// ranges (unpermuted they are 256 bytes apart: the same banks).
__device__ __forceinline__ int mask_word(int t, int c) {
    return (((2 * t + (c >> 2)) ^ (((t >> 3) & 3) << 2)) << 2) + (c & 3);
}

template <int MAXT>
__global__ __launch_bounds__(256) void b2w_kernel(B2WParams P) {
    using C = B2W<MAXT>;
    constexpr int RPT = C::RPT;
    extern __shared__ uint4 b2w_smem[];
    lds_char *smem = (lds_char *)b2w_smem;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, li = lane & 15;
    // Work order: consecutive work-groups go to the eight XCDs in turn, so with
    // a multiple of 8 column tiles XCD j takes column tiles j*nct/8 .. +nct/8-1
    // of every item, item by item; an item's split rows are then fetched into
    // one XCD's L2 once and read from there by its nct/8 tiles (otherwise
    // the tiles of an item land on different XCDs, far apart in time).
    int item = blockIdx.x, ct = blockIdx.y;
    if ((P.nct & 7) == 0) {
        const int lin = blockIdx.x + blockIdx.y * gridDim.x;
        const int ncj = P.nct >> 3, local = lin >> 3;
        item = local / ncj;
        ct = (lin & 7) * ncj + local % ncj;
    }
    const int k0 = ct * 256;

    int row_lo, row_hi;
    AdapterView ad;
    if (!resolve_chunk(P.work, item, P.m, row_lo, row_hi, ad)) return;
    const int r = ad.r;
    const int nbt = (r + 15) >> 4;
    const int rpa = 16 * (nbt <= 1 ? 1 : nbt <= 2 ? 2 : nbt <= 4 ? 4 : 8);  // the item's split row: 2 rpa bf16
    const float s = drop_scale(ad.p);
    const int nrows = row_hi - row_lo;
    const int nsb = (nrows + 31) / 32;
    const bool has_mask = P.keep != nullptr;
    auto clampb = [](uint64_t v) { return (uint32_t)(v < 0x7FFFFFF0ull ? v : 0x7FFFFFF0ull); };
    const sgpr4_t dX = make_desc(P.X + (size_t)row_lo * P.k, clampb((uint64_t)nrows * P.k * 2));
    const sgpr4_t dK = make_desc(has_mask ? P.keep + (size_t)row_lo * P.KW : P.keep,
                                 has_mask ? clampb((uint64_t)nrows * P.KW * 4) : 0u);
    const sgpr4_t dD = C::PRESPLIT
        ? make_desc(P.dss + (size_t)row_lo * P.dss_ld, clampb((uint64_t)nrows * P.dss_ld * 2))
        : make_desc(P.dS + (size_t)row_lo * P.RS, clampb((uint64_t)nrows * P.RS * 4));

    // this lane's X offsets inside sub-block 0 (4 loads of 2 rows x 512 bytes);
    // the split rows use the same rows and chunk swizzle
    uint32_t offX[4], offD[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int rr = 2 * (4 * wave + j) + (lane >> 5);
        const int c = (lane & 31) ^ swz512(rr);
        const int col = k0 + 8 * c;
        offX[j] = col < P.k ? (uint32_t)(((size_t)rr * P.k + col) * 2) : kOOBL;
        offD[j] = 8 * c < 2 * rpa ? (uint32_t)(((size_t)rr * P.dss_ld + 8 * c) * 2) : kOOBL;
    }
    auto issue = [&](int sb, int stage) {
        const uint32_t base = lds0 + stage * C::STAGE;
        const bool live = sb < nsb;
        const uint32_t xo = (uint32_t)((size_t)sb * 32 * P.k * 2);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            dma16(dX, (live && offX[j] != kOOBL) ? offX[j] + xo : kOOBL, base + (4 * wave + j) * 1024);
        // mask words: lane l fills the 16-byte slot l of the stage's mask tile
        // with words 4 h .. 4 h + 3 of tile row t, where 2 t + h = l ^ (((l >> 4) & 3) << 2)
        // (mask_word below reads them back)
        auto mask_off = [&]() {
            const int s = lane ^ (((lane >> 4) & 3) << 2);
            const int w0 = (k0 >> 5) + 4 * (s & 1);
            const int row = sb * 32 + (s >> 1);
            return (live && has_mask && w0 < P.KW && row < nrows) ? (uint32_t)(((size_t)row * P.KW + w0) * 4) : kOOBL;
        };
        if constexpr (C::PRESPLIT) {
            const uint32_t so = (uint32_t)((size_t)sb * 32 * P.dss_ld * 2);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = sb * 32 + 2 * (4 * wave + j) + (lane >> 5);
                dma16(dD, (live && row < nrows && offD[j] != kOOBL) ? offD[j] + so : kOOBL,
                      base + C::SPL_OFF + (4 * wave + j) * 1024);
            }
            // wave 0: the mask words; the others a dummy load into the kibibyte past them
            dma16(dK, wave == 0 ? mask_off() : kOOBL, base + C::MASK_OFF + (wave == 0 ? 0 : 1024));
        } else {
#pragma unroll
            for (int q0 = 0; q0 < C::NPW; ++q0) {
                const int q = wave * C::NPW + q0;
                const uint32_t dst = base + C::X_BYTES + q * 1024;
                uint32_t off = kOOBL;
                if (q == 0) {
                    off = mask_off();
                } else if (q < C::NA) {
                    const int f = (q - 1) * 256 + 4 * lane;
                    const int row = sb * 32 + f / RPT, col = f % RPT;
                    if (live && row < nrows && col < r && col < P.RS) off = (uint32_t)(((size_t)row * P.RS + col) * 4);
                }
                dma16(q == 0 ? dK : dD, off, dst);
            }
        }
    };

    // The main loop is instantiated per number of 16-rank blocks the chunk's
    // adapter needs (1, 2, 4 or 8, at most MAXT), so the MFMA stream has no
    // per-block branches and the accumulators stay in fixed registers.
    constexpr int NPS = 4 + C::NPW;  // loads per wave per stage
    auto body = [&](auto nb_c) {
        constexpr int NB = decltype(nb_c)::value;
        f32x4_t acc[4][NB];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int y = 0; y < NB; ++y) acc[x][y] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < C::NST - 1; ++q) issue(q, q);
        wait_vmcnt<NPS * (C::NST - 2)>();
        __syncthreads();
        int stage = 0, lstage = C::NST - 1;
        for (int sb = 0; sb < nsb; ++sb) {
            issue(sb + C::NST - 1, lstage);
            const lds_char *xt = smem + stage * C::STAGE;
            const uint32_t *mk = (const uint32_t *)(xt + C::MASK_OFF);
            // dS operand (N = rank): rows 8g .. 8g+7 of rank 16 bt + li, times s
            uint4 bhi[NB], blo[NB];
            if constexpr (C::PRESPLIT) {
#pragma unroll
                for (int bt = 0; bt < NB; ++bt) {
                    bhi[bt] = tile_rows8(xt + C::SPL_OFF, 8 * g, bt, lane);
                    blo[bt] = tile_rows8(xt + C::SPL_OFF, 8 * g, NB + bt, lane);
                }
            } else {
                const float *ds = (const float *)(xt + C::DS_OFF);
#pragma unroll
                for (int bt = 0; bt < NB; ++bt) {
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = s * ds[(8 * g + e) * RPT + 16 * bt + li];
                    split_frag(v, bhi[bt], blo[bt]);
                }
            }
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int cb = 4 * wave + mb;
                uint4 xf = tile_rows8(xt, 8 * g, cb, lane);
                if (has_mask) {
                    const int bit = 16 * (cb & 1) + li;
                    uint32_t mm[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t w0 = mk[mask_word(8 * g + 2 * q, cb >> 1)];
                        const uint32_t w1 = mk[mask_word(8 * g + 2 * q + 1, cb >> 1)];
                        // each keep bit sign-extended to a whole word, the pair
                        // merged into one 16-bit mask per element (3 instructions)
                        const uint32_t e0 = (uint32_t)__builtin_amdgcn_sbfe((int)w0, bit, 1);
                        const uint32_t e1 = (uint32_t)__builtin_amdgcn_sbfe((int)w1, bit, 1);
                        mm[q] = (e0 & 0x0000FFFFu) | (e1 & 0xFFFF0000u);
                    }
                    xf = make_uint4(xf.x & mm[0], xf.y & mm[1], xf.z & mm[2], xf.w & mm[3]);
                }
#pragma unroll
                for (int bt = 0; bt < NB; ++bt) {
                    acc[mb][bt] = mfma16x16x32(xf, bhi[bt], acc[mb][bt]);
                    acc[mb][bt] = mfma16x16x32(xf, blo[bt], acc[mb][bt]);
                }
            }
            wait_vmcnt<NPS * (C::NST - 2)>();
            __syncthreads();
            stage = stage == C::NST - 1 ? 0 : stage + 1;
            lstage = lstage == C::NST - 1 ? 0 : lstage + 1;
        }
        wait_vmcnt<0>();
        // this item's partial: columns ct*256 .. +255 of its [nct*256][16 NB]
        // block (the item's slot holds nct*256*RPT floats)
        float *pp = P.part + (size_t)item * P.nct * 256 * RPT + (size_t)ct * 256 * (16 * NB);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int bt = 0; bt < NB; ++bt)
#pragma unroll
                for (int v = 0; v < 4; ++v) pp[((4 * wave + mb) * 16 + 4 * g + v) * (16 * NB) + 16 * bt + li] = acc[mb][bt][v];
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    using I8 = std::integral_constant<int, 8>;
    if constexpr (MAXT == 1) {
        body(I1{});
    } else if constexpr (MAXT == 2) {
        if (nbt <= 1) body(I1{});
        else body(I2{});
    } else if constexpr (MAXT == 4) {
        if (nbt <= 1) body(I1{});
        else if (nbt <= 2) body(I2{});
        else body(I4{});
    } else {
        if (nbt <= 1) body(I1{});
        else if (nbt <= 2) body(I2{});
        else if (nbt <= 4) body(I4{});
        else body(I8{});
    }
}

// dA of every adapter from the single-pass kernel's partials: an item of
// adapter a holds a [columns][RPa] block, RPa = 16 * (1, 2, 4 or 8, the
// 16-rank blocks its pass ran).  Thread t of work-group (x, a) owns float4
// 256 x + t of that block and adds that float4 of each of a's work items in
// work-item order (8 items' loads in flight at a time); adapters without
// rows get zeros.  Work-groups past an adapter's block exit at once.
struct DAReduceParams {
    const float *part;
    int k, nct, RPT;
    RowWork work;
    int items;                // single: number of items; multi: the table's capacity
    const int32_t *ad_items;  // multi: the router's per-adapter item counts
};

__global__ __launch_bounds__(256) void da_reduce_kernel(DAReduceParams P) {
    __shared__ int s_ad[1024];
    const int a = blockIdx.y;
    const bool single = P.work.chunks == nullptr;
    AdapterView ad;
    int cnt;
    if (single) {
        ad = P.work.single;
        cnt = P.items;
    } else {
        ad = load_adapter(P.work.adapters, a);
        cnt = P.ad_items[a];
    }
    const int r = ad.r;
    if (r < 1 || r > P.work.r_cap || ad.dA == nullptr) return;  // uniform over the work-group
    const int nbt = (r + 15) >> 4;
    const int rpa = 16 * (nbt <= 1 ? 1 : nbt <= 2 ? 2 : nbt <= 4 ? 4 : 8);
    if ((size_t)blockIdx.x * 256 * 4 >= (size_t)P.k * rpa) return;  // past this adapter's block
    const int f = blockIdx.x * 256 + threadIdx.x;
    const int col = 4 * f / rpa, r0 = 4 * f % rpa;
    const bool active = col < P.k && r0 < r;
    const size_t istride = (size_t)P.nct * 256 * P.RPT / 4;  // float4s per item slot
    const float4 *src = (const float4 *)P.part + f;
    const int nit = cnt <= 0 ? 0 : single ? P.items : min(P.work.chunk_count[0], P.items);
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    // the work items' adapters, a window of up to 1024 at a time in LDS; each
    // thread walks the window in order and loads 8 of a's items at once
    for (int base = 0; base < nit; base += 1024) {
        const int nw = min(1024, nit - base);
        __syncthreads();
        for (int i = threadIdx.x; i < nw; i += 256) s_ad[i] = single ? a : P.work.chunks[base + i].adapter;
        __syncthreads();
        int i = 0;
        while (i < nw) {
            int id[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                while (i < nw && s_ad[i] != a) ++i;
                id[u] = i < nw ? base + i : -1;
                if (i < nw) ++i;
            }
            float4 t[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                t[u] = (active && id[u] >= 0) ? src[(size_t)id[u] * istride] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                sum.x += t[u].x;
                sum.y += t[u].y;
                sum.z += t[u].z;
                sum.w += t[u].w;
            }
        }
    }
    if (!active) return;
    const float v[4] = {sum.x, sum.y, sum.z, sum.w};
    uint16_t *dst = ad.dA + (size_t)col * r + r0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (r0 + e < r) dst[e] = (uint16_t)f32_to_bf16_rne(v[e]);
}

// ----- B1 streaming (ranks <= 32 per rank tile).  Work-group = one row group
// (rows of one adapter) x C1 = 256*CW columns; rows go in sub-blocks of 32
// through a 3-stage ring of direct-to-LDS loads (dY as CW swizzled 256-column
// sub-tiles, plus the 32 rows of S).  Wave w owns the 16-column blocks 4*CW*w .. +4*CW-1:
// it accumulates dB = alpha S^T dY for them over all the group's rows, and
// its share of dS = alpha dY B^T for each sub-block; the four shares meet in
// LDS and are summed in wave order into one dS partial per column tile.  The
// B fragments of the wave's columns stay in registers.
constexpr int B1V_SUB = 32 * 512;  // one 32-row x 256-column sub-tile

template <int CW, int MAXT, int NST>
__global__ __launch_bounds__(256) void b1v_kernel(B1Params P) {
    constexpr int RL = 16 * MAXT;
    constexpr int SY = CW * B1V_SUB;        // dY bytes per stage
    constexpr int STAGE = SY + 32 * 32 * 4;  // + 32 rows of S (up to 32 fp32 each)
    constexpr int NB = 4 * CW;               // 16-column blocks per wave
    constexpr int NQ = 2 * CW;               // 32-column k-steps per wave (dS)
    constexpr int NDMA = 4 * CW + 1;         // direct-to-LDS loads per wave per stage
    extern __shared__ uint4 b1v_smem[];
    lds_char *smem = (lds_char *)b1v_smem;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    // [NRED][4 waves][32 rows][RLP]: double-buffered for RL = 16; for RL = 32 one
    // buffer and a second barrier per sub-block, so two work-groups fit a CU.
    // Rows are RL + 4 floats apart, so the four 4-row groups of a wave's
    // stores (rows 4g + v) fall on four different 16-bank ranges.
    constexpr int NRED = MAXT == 1 ? 2 : 1;
    constexpr int RLP = RL + 4;
    float *red = (float *)(smem + NST * STAGE);

    // Work order (mixed adapters): consecutive work-groups go to the eight XCDs
    // in turn; with a multiple of 8 column tiles, within each rank tile XCD j
    // takes column tiles j*CT/8 .. +CT/8-1 of every row group, group by group,
    // so a row group's S rows (r_max floats each) are fetched into one XCD's L2
    // once for its CT/8 tiles instead of once per tile.  The single-adapter
    // form keeps the grid order (measured faster there).
    int grp = blockIdx.x, ct = blockIdx.y;
    if ((gridDim.y & 7) == 0 && P.work.chunks != nullptr &&
        (uint64_t)gridDim.x * gridDim.y < (uint64_t(1) << 31)) {
        const int p = blockIdx.x + gridDim.x * blockIdx.y;  // within the rank tile's plane
        const int ncj = gridDim.y >> 3, local = p >> 3;
        grp = local / ncj;
        ct = (p & 7) * ncj + local % ncj;
    }
    int row_lo, row_hi;
    AdapterView ad;
    if (!resolve_chunk(P.work, grp, P.m, row_lo, row_hi, ad)) return;
    const int r = ad.r;
    const float alpha = ad.alpha;
    const int n0 = ct * 256 * CW;
    const int tid = threadIdx.x, lane = tid & 63;
    // rank tile (tiled launches, RL = 32): ranks r0 .. r0+31; S rows staged as
    // 32 floats (else whole RS-float rows, r0 = 0)
    const int r0 = P.tiled ? (int)blockIdx.z * RL : 0;
    const int sst = P.tiled ? 32 : P.RS;
    float *dsp = P.dSpart + (size_t)ct * P.m * P.RS;
    if (r0 >= r) {
        // no ranks here; with one column tile B1 writes dS itself, whose
        // columns past r are zero (with several, the finishing sum writes them)
        if (gridDim.y == 1)
            for (int i = tid; i < (row_hi - row_lo) * RL; i += 256) {
                const int rr = i / RL, cc = r0 + i % RL;
                if (cc < P.RS) dsp[(size_t)(row_lo + rr) * P.RS + cc] = 0.f;
            }
        return;
    }
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, li = lane & 15;
    const int nrows = row_hi - row_lo;
    const int nsb = (nrows + 31) / 32;
    // host guarantees nrows * n * 2 < 2^31
    const sgpr4_t dYd = make_desc(P.dY + (size_t)row_lo * P.n, (uint32_t)((uint64_t)nrows * P.n * 2));
    const sgpr4_t dSd = make_desc(P.S + (size_t)row_lo * P.RS, (uint32_t)((uint64_t)nrows * P.RS * 4));

    // dY: instruction j of a sub-tile writes LDS rows 2(4w+j), +1 (512 B each);
    // LDS chunk (lane & 31) of row rr holds global chunk (lane & 31) ^ swz512(rr)
    uint32_t offY[CW][4];
#pragma unroll
    for (int t = 0; t < CW; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = 2 * (4 * wave + j) + (lane >> 5);
            const int col = n0 + 256 * t + 8 * ((lane & 31) ^ swz512(rr));
            offY[t][j] = col < P.n ? (uint32_t)(rr * P.n + col) * 2u : kOOBL;
        }
    const uint32_t sbb = (uint32_t)(32 * P.RS * 4);  // S bytes per sub-block
    auto issue = [&](int sb, int stage) {  // sub-blocks past the last read zeros
        const uint32_t base = lds0 + stage * STAGE;
        const bool live = sb < nsb;
        const uint32_t yo = live ? (uint32_t)sb * 32u * (uint32_t)P.n * 2u : 0u;
#pragma unroll
        for (int t = 0; t < CW; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                dma16(dYd, (!live || offY[t][j] == kOOBL) ? kOOBL : offY[t][j] + yo,
                      base + t * B1V_SUB + (4 * wave + j) * 1024);
        if (P.tiled) {
            // wave w: rows 8w + lane/8, 16-byte chunk lane % 8 of the tile's 32 columns
            const int row = 8 * wave + (lane >> 3), cc = r0 + 4 * (lane & 7);
            dma16(dSd, (live && cc < P.RS) ? (uint32_t)(((size_t)sb * 32 + row) * P.RS + cc) * 4u : kOOBL,
                  base + SY + wave * 1024);
        } else {
            const uint32_t b = (uint32_t)wave * 1024 + lane * 16;
            dma16(dSd, (live && b < sbb) ? (uint32_t)sb * sbb + b : kOOBL, base + SY + wave * 1024);
        }
    };

    // B fragments for dS: rank 16bt + li, columns n0 + 64CW w + 32q + 8g .. +7
    uint4 bfr[NQ][MAXT];
    {
        const __amdgpu_buffer_rsrc_t rB = make_rsrc(ad.B, (size_t)r * P.n * 2);
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int bt = 0; bt < MAXT; ++bt) {
                const int rank = r0 + 16 * bt + li;
                const int col = n0 + 64 * CW * wave + 32 * q + 8 * g;
                const uint32_t off = (rank < r && col < P.n) ? (uint32_t)(rank * P.n + col) * 2u : kOOB;
                bfr[q][bt] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rB, off, 0, 0));
            }
    }

    f32x4_t accB[MAXT][NB];
#pragma unroll
    for (int a = 0; a < MAXT; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) accB[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int q = 0; q < NST - 1; ++q) issue(q, q);
    wait_vmcnt<NDMA * (NST - 2)>();
    __syncthreads();
    // sum of the four waves' dS shares of sub-block sb (after the barrier)
    // thread t handles row t / 8 of the sub-block, columns t % 8, +8, ...
    auto flush_ds = [&](int sb) {
        const float *rd = red + (sb % NRED) * (4 * 32 * RLP);
        const int rr = tid >> 3, rs = row_lo + sb * 32;
        if (rs + rr >= row_hi) return;
        float *drow = dsp + (size_t)(rs + rr) * P.RS;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int cl = (tid & 7) + 8 * j, cc = r0 + cl;
            if (cl >= RL || cc >= P.RS) break;
            float v = rd[(0 * 32 + rr) * RLP + cl];
            v += rd[(1 * 32 + rr) * RLP + cl];
            v += rd[(2 * 32 + rr) * RLP + cl];
            v += rd[(3 * 32 + rr) * RLP + cl];
            drow[cc] = cc < r ? v * alpha : 0.f;
        }
    };
    int stage = 0, lstage = NST - 1;
    for (int sb = 0; sb < nsb; ++sb) {
        issue(sb + NST - 1, lstage);
        const lds_char *yt = smem + stage * STAGE;
        const float *st = (const float *)(yt + SY);

        // ---- dS share: 32 rows x rank over the wave's 64*CW columns
        f32x4_t accS[2][MAXT];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < MAXT; ++b) accS[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int blk = NB * wave + 2 * q;  // first 16-column block of the step
            const lds_char *sub = yt + (blk >> 4) * B1V_SUB;
            const int chunk = 2 * (blk & 15) + g;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const uint4 af = *(const uint4 *)(sub + swz512_off(16 * rb + li, chunk));
#pragma unroll
                for (int bt = 0; bt < MAXT; ++bt) accS[rb][bt] = mfma16x16x32(af, bfr[q][bt], accS[rb][bt]);
            }
        }
        float *rw = red + (sb % NRED) * (4 * 32 * RLP) + wave * 32 * RLP;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int bt = 0; bt < MAXT; ++bt)
#pragma unroll
                for (int v = 0; v < 4; ++v) rw[(16 * rb + 4 * g + v) * RLP + 16 * bt + li] = accS[rb][bt][v];

        // ---- dB: rank x the wave's columns, K = the 32 rows
        uint4 ahi[MAXT], alo[MAXT];
#pragma unroll
        for (int bt = 0; bt < MAXT; ++bt) {
            float v[8];
            const int rr = 16 * bt + li;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // in-bounds for every lane (rows < 32, RS and rr < 32): read, then select
                const float sv = st[(8 * g + e) * sst + rr];
                v[e] = r0 + rr < r ? alpha * sv : 0.f;
            }
            split_frag(v, ahi[bt], alo[bt]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int blk = NB * wave + b;
            const uint4 yf = tile_rows8(yt + (blk >> 4) * B1V_SUB, 8 * g, blk & 15, lane);
#pragma unroll
            for (int bt = 0; bt < MAXT; ++bt) {
                accB[bt][b] = mfma16x16x32(ahi[bt], yf, accB[bt][b]);
                accB[bt][b] = mfma16x16x32(alo[bt], yf, accB[bt][b]);
            }
        }
        wait_vmcnt<NDMA * (NST - 2)>();
        __syncthreads();
        flush_ds(sb);
        if constexpr (NRED == 1) __syncthreads();  // the next sub-block rewrites red
        stage = stage == NST - 1 ? 0 : stage + 1;
        lstage = lstage == NST - 1 ? 0 : lstage + 1;
    }
    wait_vmcnt<0>();

    float *dbp = P.dBpart + (size_t)grp * P.RS * P.n;
#pragma unroll
    for (int bt = 0; bt < MAXT; ++bt)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int col = n0 + 16 * (NB * wave + b) + li;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int rr = r0 + 16 * bt + 4 * g + v;
                if (rr < r && col < P.n) dbp[(size_t)rr * P.n + col] = accB[bt][b][v];
            }
        }
}

// ===========================================================================
// Per-adapter gradient reduction: sum the chunk partials that belong to the
// adapter, in chunk order, and write bf16 (zeros if the adapter has no rows).
// ===========================================================================
struct GradReduceParams {
    const float *part;
    int which;  // 0: dB [chunk][RS][n] -> r x n; 1: dA [chunk][k][RS] -> k x r
    int m, k, n, RS;
    RowWork work;
    int chunk_cap;
};

__device__ __forceinline__ void grad_reduce_block(const GradReduceParams &P, int a, int bx, int gx) {
    __shared__ float red[4][64];
    AdapterView ad;
    if (P.work.chunks == nullptr) {
        ad = P.work.single;
    } else {
        ad = load_adapter(P.work.adapters, a);
    }
    const int r = ad.r;
    if (r < 1 || r > P.work.r_cap) return;
    uint16_t *outp = P.which == 0 ? ad.dB : ad.dA;
    if (outp == nullptr) return;
    const int rows_out = P.which == 0 ? r : P.k;
    const int cols_out = P.which == 0 ? P.n : r;
    const size_t total = (size_t)rows_out * cols_out;
    const size_t chunk_stride = (size_t)P.RS * (P.which == 0 ? P.n : P.k);
    const size_t row_stride = P.which == 0 ? (size_t)P.n : (size_t)P.RS;
    int nch;
    if (P.work.chunks == nullptr) nch = (P.m + P.work.rows_per_chunk - 1) / P.work.rows_per_chunk;
    else nch = min(P.work.chunk_count[0], P.chunk_cap);

    // 64 outputs per work-group pass; wave pg sums chunks pg, pg+4, ...
    const int t = threadIdx.x, pg = t >> 6, c = t & 63;
    for (size_t base = (size_t)bx * 64; base < total; base += (size_t)gx * 64) {
        const size_t e = base + c;
        float acc = 0.f;
        if (e < total) {
            const size_t ro = e / cols_out, co = e - ro * cols_out;
            const float *src = P.part + ro * row_stride + co;
#pragma unroll 4
            for (int ch = pg; ch < nch; ch += 4) {
                if (P.work.chunks != nullptr && P.work.chunks[ch].adapter != a) continue;
                acc += src[(size_t)ch * chunk_stride];
            }
        }
        __syncthreads();
        red[pg][c] = acc;
        __syncthreads();
        if (pg == 0 && e < total) {
            const float v = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
            outp[e] = (uint16_t)f32_to_bf16_rne(v);
        }
    }
}

__global__ __launch_bounds__(256) void grad_reduce_kernel(GradReduceParams P) {
    grad_reduce_block(P, blockIdx.y, blockIdx.x, gridDim.x);
}

// ===========================================================================
// B1's finishing sums, one launch.  Work-groups [0, ds_wgs): dS of each row
// group = the column tiles' partials added in tile order, ranks below the
// group's adapter rank only (zeros past it up to RS); the rest: dB of each
// adapter = its row groups' partials added in group order, a float4 per
// thread with 8 groups' loads in flight (work-groups past the adapter's r x n
// exit at once; an adapter with no rows gets zeros).
// ===========================================================================
struct B1FinishParams {
    const float *dspart;  // [nparts][m][RS] (nparts == 1: dS itself)
    int nparts;
    float *ds;
    uint16_t *dss;        // optional: rows of [hi | lo] of s*dS for the dA pass and the dX epilogue
    int dss_ld;
    int m, n, RS;
    const float *dbpart;  // [group][RS][n]
    RowWork work;         // B1 row groups (router table 2, or rows_per_chunk rows)
    int groups;           // single: number of row groups; multi: the table's capacity
    int ds_wpg;           // dS work-groups per row group (0: no dS pass)
    int db_gx;            // dB work-groups per adapter
};

__global__ __launch_bounds__(256) void b1_finish_kernel(B1FinishParams P) {
    __shared__ int s_ad[1024];
    const int tid = threadIdx.x;
    const bool single = P.work.chunks == nullptr;
    const int ds_wgs = P.groups * P.ds_wpg;
    if ((int)blockIdx.x < ds_wgs) {
        const int grp = blockIdx.x / P.ds_wpg, sub = blockIdx.x - grp * P.ds_wpg;
        int row_lo, row_hi;
        AdapterView ad;
        if (!resolve_chunk(P.work, grp, P.m, row_lo, row_hi, ad)) return;
        const int r = min(ad.r, P.RS);
        // the split row of this group's adapter: hi of ranks 0 .. rpa-1, then
        // their lo parts (rpa = 16 x the power-of-two 16-rank block count the
        // dA pass runs for this rank); ranks past r are zero
        const int nbt = (ad.r + 15) >> 4;
        const int rpa = P.dss ? 16 * (nbt <= 1 ? 1 : nbt <= 2 ? 2 : nbt <= 4 ? 4 : 8) : 0;
        const float s = drop_scale(ad.p);
        const int W = max(P.RS, rpa);  // columns this pass covers per row
        const size_t ps = (size_t)P.m * P.RS;
        const int total = (row_hi - row_lo) * W;
        for (int e = sub * 256 + tid; e < total; e += P.ds_wpg * 256) {
            const int lr = e / W, rr = e - lr * W;
            const int row = row_lo + lr;
            const size_t idx = (size_t)row * P.RS + rr;
            float v = 0.f;
            if (rr < r) {
                const float *src = P.dspart + idx;
                if (P.nparts == 1) {
                    v = *src;
                } else {
                    int q = 0;
                    for (; q + 8 <= P.nparts; q += 8) {
                        float t[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) t[u] = src[(size_t)(q + u) * ps];
#pragma unroll
                        for (int u = 0; u < 8; ++u) v += t[u];
                    }
                    for (; q < P.nparts; ++q) v += src[(size_t)q * ps];
                }
            }
            if (P.nparts > 1 && rr < P.RS) P.ds[idx] = v;
            if (rr < rpa) {
                uint32_t hi, lo;
                split_bf16(s * v, hi, lo);
                uint16_t *drow = P.dss + (size_t)row * P.dss_ld;
                drow[rr] = (uint16_t)hi;
                drow[rpa + rr] = (uint16_t)lo;
            }
        }
        return;
    }
    const int y = blockIdx.x - ds_wgs;
    const int a = y / P.db_gx, bx = y - a * P.db_gx;
    AdapterView ad;
    if (single) {
        if (a != 0) return;
        ad = P.work.single;
    } else {
        if (a >= P.work.num_adapters) return;
        ad = load_adapter(P.work.adapters, a);
    }
    const int r = ad.r;
    if (r < 1 || r > P.work.r_cap || ad.dB == nullptr) return;
    if ((size_t)bx * 256 * 4 >= (size_t)r * P.n) return;  // past this adapter's r x n
    const int f = bx * 256 + tid;
    const bool active = (size_t)4 * f < (size_t)r * P.n;
    const size_t gstride = (size_t)P.RS * P.n / 4;  // float4s per group partial
    const float4 *src = (const float4 *)P.dbpart + f;
    const int ngr = single ? P.groups : min(P.work.chunk_count[0], P.groups);
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int base = 0; base < ngr; base += 1024) {
        const int nw = min(1024, ngr - base);
        __syncthreads();
        for (int i = tid; i < nw; i += 256) s_ad[i] = single ? a : P.work.chunks[base + i].adapter;
        __syncthreads();
        int i = 0;
        while (i < nw) {
            int id[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                while (i < nw && s_ad[i] != a) ++i;
                id[u] = i < nw ? base + i : -1;
                if (i < nw) ++i;
            }
            float4 t[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                t[u] = (active && id[u] >= 0) ? src[(size_t)id[u] * gstride] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                sum.x += t[u].x;
                sum.y += t[u].y;
                sum.z += t[u].z;
                sum.w += t[u].w;
            }
        }
    }
    if (!active) return;
    const float v[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) ad.dB[4 * (size_t)f + e] = (uint16_t)f32_to_bf16_rne(v[e]);
}

// ===========================================================================
// Mask alone: one thread per 32-bit word (32 elements = 4 Philox blocks).
// ===========================================================================
__global__ __launch_bounds__(256) void mask_kernel(uint64_t seed, uint64_t offset, int m, int k,
                                                   uint32_t T, uint32_t *bits) {
    const int KW = (k + 31) >> 5;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (size_t)m * KW) return;
    const int row = (int)(idx / KW), w = (int)(idx - (size_t)row * KW);
    const uint64_t base = offset + (uint64_t)row * (uint64_t)k;
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c0 = w * 32 + q * 8;
        if (c0 < k) word |= keep_byte(base + (uint64_t)c0, seed, T) << (8 * q);
    }
    bits[idx] = word;
}

// ===========================================================================
// Launchers
// ===========================================================================
static inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

static hipError_t finish_launch(int slot, hipStream_t stream) {
    hipError_t e = hipGetLastError();
    prof_end(slot, stream);
    return e;
}

hipError_t launch_router(const int64_t *seg_off, const int32_t *seg_adapter, int nseg, int m,
                         const lora_adapter *adapters, int nad, int r_cap, ChunkEntry *t_f1,
                         int32_t *c_f1, int cap_f1, ChunkEntry *t_bwd, int32_t *c_bwd, int rows_bwd, int cap_bwd,
                         ChunkEntry *t_b1, int32_t *c_b1, int rows_b1, int cap_b1, hipStream_t stream,
                         int32_t *ad_items) {
    RouterTables T;
    T.tab[0] = RouterTable{t_f1, c_f1, kF1Rows, cap_f1};
    T.tab[1] = RouterTable{t_bwd, c_bwd, rows_bwd, cap_bwd};
    T.tab[2] = RouterTable{t_b1, c_b1, t_b1 != nullptr ? rows_b1 : 0, cap_b1};
    (void)hipGetLastError();
    const int slot = prof_begin("router", stream);
    hipLaunchKernelGGL(router_kernel, dim3(1), dim3(1024), 0, stream, seg_off, seg_adapter, nseg, m,
                       adapters, nad, r_cap, T, ad_items);
    return finish_launch(slot, stream);
}

// Number of 16-wide rank blocks a kernel instance is built for (power of 2).
static int rank_blocks(int r_lds) {
    const int nb = r_lds / 16;
    int p = 1;
    while (p < nb) p <<= 1;
    return p;
}

template <typename Kernel, typename Params>
static void launch_with_lds(Kernel kernel, dim3 grid, size_t lds, hipStream_t stream, const Params &P,
                            int threads = 256) {
    if (lds > 64 * 1024) (void)hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(kernel, grid, dim3(threads), lds, stream, P);
}

static int r_lds_of(const AdapterSource &src) {
    const int rc = src.table ? src.r_cap : src.r;
    return ((rc + 15) / 16) * 16;
}

hipError_t launch_f1(const void *X, int m, int k, const AdapterSource &src, int chunk_cap,
                     uint64_t seed, uint64_t offset, uint32_t *keep_bits, float *out, int RS,
                     int KS, int ksl, hipStream_t stream, uint16_t *s2, int s2_rp) {
    F1Params P;
    P.s2 = s2;
    P.s2_rp = s2_rp;
    P.X = (const uint16_t *)X;
    P.m = m;
    P.k = k;
    P.work = make_work(src, kTabF1);
    P.seed = seed;
    P.offset = offset;
    P.keep_bits = keep_bits;
    P.out = out;
    P.RS = RS;
    P.ksl = ksl;
    P.KW = (k + 31) / 32;
    P.r_lds = r_lds_of(src);
    // A slab: about 20 KiB of LDS so several work-groups share a CU
    const int slab_cols = std::max(kF1KSub, (20480 / (P.r_lds * 2)) / kF1KSub * kF1KSub);
    P.slab = std::min(ksl, slab_cols);
    const size_t lds = (size_t)P.r_lds * (P.slab + 8) * sizeof(uint16_t);
    (void)hipGetLastError();
    const int slot = prof_begin("f1_mask_down", stream);
    if (f1_streaming(P.r_lds, k)) {
        // streaming form: 4 work-groups of 16 rows per chunk, all of k each,
        // times the rank tiles
        const dim3 g4(4 * chunk_cap, rank_tiles(P.r_lds));
        if (P.r_lds <= 16) {
            launch_with_lds(f1s_kernel<1>, g4, (size_t)F1S_WAVES * 2 * F1S_UNIT * 16 * 2, stream, P, 64 * F1S_WAVES);
        } else if (f1_rank64(P.r_lds, src.table != nullptr)) {
            // one adapter with an even number of 32-rank tiles: half as many
            // passes over X in tiles of 64 (one work-group per CU; measured
            // faster at 64 and 128 ranks, slower at 96)
            launch_with_lds(f1s_kernel<4>, dim3(4 * chunk_cap, (P.r_lds + 63) / 64),
                            (size_t)F1S_WAVES * 1 * F1S_UNIT * 64 * 2, stream, P, 64 * F1S_WAVES);
        } else {
            launch_with_lds(f1s_kernel<2>, g4, (size_t)F1S_WAVES * 1 * F1S_UNIT * 32 * 2, stream, P, 64 * F1S_WAVES);
        }
        return finish_launch(slot, stream);
    }
    const dim3 grid(chunk_cap, KS);
    switch (rank_blocks(P.r_lds)) {
    case 1: launch_with_lds(f1_kernel<1>, grid, lds, stream, P); break;
    case 2: launch_with_lds(f1_kernel<2>, grid, lds, stream, P); break;
    case 4: launch_with_lds(f1_kernel<4>, grid, lds, stream, P); break;
    case 8: launch_with_lds(f1_kernel<8>, grid, lds, stream, P); break;
    default: launch_with_lds(f1_kernel<16>, grid, lds, stream, P); break;
    }
    return finish_launch(slot, stream);
}

hipError_t launch_f1w(const void *X, int m, int k, const AdapterSource &src, int chunk_cap, uint64_t seed,
                      uint64_t offset, uint32_t *keep_bits, float *S, int RS, float *part, int KS, int ksl,
                      hipStream_t stream, uint16_t *s2, int s2_rp) {
    F1WParams P;
    P.X = (const uint16_t *)X;
    P.m = m;
    P.k = k;
    P.work = make_work(src, kTabF1);
    P.seed = seed;
    P.offset = offset;
    P.keep_bits = keep_bits;
    P.KW = (k + 31) / 32;
    P.S = S;
    P.RS = RS;
    P.part = part;
    P.ksl = ksl;
    P.KS = KS;
    P.s2 = s2;
    P.s2_rp = s2_rp;
    const int mt = f1w_blocks(r_lds_of(src));
    (void)hipGetLastError();
    int slot = prof_begin("f1_mask_down", stream);
    const dim3 grid((unsigned)chunk_cap, (unsigned)KS);
    if (mt == 4) launch_with_lds(f1w_kernel<4>, grid, (size_t)F1W<4>::LDS, stream, P);
    else launch_with_lds(f1w_kernel<8>, grid, (size_t)F1W<8>::LDS, stream, P);
    hipError_t e = finish_launch(slot, stream);
    if (e != hipSuccess || KS == 1) return e;
    slot = prof_begin("sum_s_partials", stream);
    const int width = std::max(RS, s2 != nullptr ? s2_rp : 0);
    hipLaunchKernelGGL(f1_reduce_kernel, dim3((unsigned)chunk_cap, (unsigned)cdiv(kF1Rows * width, 256)), dim3(256), 0,
                       stream, P, 16 * mt);
    return finish_launch(slot, stream);
}

hipError_t launch_sum_partials(const float *part, int nparts, size_t part_stride, size_t count,
                               float *out, const char *name, hipStream_t stream) {
    if (count == 0) return hipSuccess;
    (void)hipGetLastError();
    const int slot = prof_begin(name, stream);
    const size_t blocks = (count + 255) / 256;
    hipLaunchKernelGGL(sum_partials_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part,
                       nparts, part_stride, count, out);
    return finish_launch(slot, stream);
}

size_t b1_lds_bytes(int C1, int r_lds) {
    return (size_t)r_lds * (C1 + 8) * 2 + (size_t)64 * (C1 + 8) * 2 + (size_t)r_lds * 68 * 4;
}
size_t b2_lds_bytes(int C2, int r_lds) { return (size_t)C2 * 72 * 2 + (size_t)r_lds * 68 * 4; }

hipError_t launch_b1(const void *dY, const float *S, int m, int n, int RS, const AdapterSource &src,
                     const B1Shape &sh, float *dSpart, float *dBpart, hipStream_t stream) {
    B1Params P;
    P.dY = (const uint16_t *)dY;
    P.S = S;
    P.m = m;
    P.n = n;
    P.RS = RS;
    P.work = make_work(src, kTabB1);
    P.work.rows_per_chunk = sh.rows;
    P.dSpart = dSpart;
    P.dBpart = dBpart;
    P.r_lds = r_lds_of(src);
    P.tiled = P.r_lds > 32;
    (void)hipGetLastError();
    const int slot = prof_begin("b1_ds_db", stream);
    const dim3 grid(sh.slots, sh.CT, sh.streaming ? rank_tiles(P.r_lds) : 1);
    if (sh.streaming) {
        if (sh.cw != 1) return hipErrorInvalidValue;  // the streaming kernel is built for 256-column tiles
        if (P.tiled && RS % 4 != 0) return hipErrorInvalidValue;  // tiles stage 16-byte row pieces
        const int rl = P.r_lds <= 16 ? 16 : 32;
        // ring depth 3: two stages in flight, two work-groups per CU
        auto lds_of = [&](int nst) {
            return (size_t)nst * (sh.cw * B1V_SUB + 32 * 32 * 4) + (size_t)(rl == 16 ? 2 : 1) * 4 * 32 * (rl + 4) * 4;
        };
        if (rl == 16) launch_with_lds(b1v_kernel<1, 1, 3>, grid, lds_of(3), stream, P);
        else launch_with_lds(b1v_kernel<1, 2, 3>, grid, lds_of(3), stream, P);
    } else {
        const size_t lds = b1_lds_bytes(sh.C1, P.r_lds);
        if (sh.C1 == 256) {
            switch (rank_blocks(P.r_lds)) {
            case 1: launch_with_lds(b1_kernel<256, 1>, grid, lds, stream, P); break;
            case 2: launch_with_lds(b1_kernel<256, 2>, grid, lds, stream, P); break;
            case 4: launch_with_lds(b1_kernel<256, 4>, grid, lds, stream, P); break;
            default: launch_with_lds(b1_kernel<256, 8>, grid, lds, stream, P); break;
            }
        } else {
            launch_with_lds(b1_kernel<128, 16>, grid, lds, stream, P);
        }
    }
    return finish_launch(slot, stream);
}

hipError_t launch_b2(const void *X, const uint32_t *keep, const float *dS, int m, int k, int RS, int rows,
                     const AdapterSource &src, int chunk_cap, int C2, float *dApart,
                     hipStream_t stream) {
    B2Params P;
    P.X = (const uint16_t *)X;
    P.keep = keep;
    P.dS = dS;
    P.m = m;
    P.k = k;
    P.RS = RS;
    P.KW = (k + 31) / 32;
    P.work = make_work(src, kTabBwd);
    P.work.rows_per_chunk = rows;
    P.dApart = dApart;
    P.r_lds = r_lds_of(src);
    P.tiled = P.r_lds > 32;
    const size_t lds = b2_lds_bytes(C2, P.r_lds);
    (void)hipGetLastError();
    const int slot = prof_begin("b2_da", stream);
    const bool streaming = C2 == 256 && bwd_streaming(P.r_lds, RS);
    const dim3 grid(chunk_cap, cdiv(k, C2), streaming ? rank_tiles(P.r_lds) : 1);
    if (streaming) {
        const size_t slds = (size_t)B2S_NST * B2S_STAGE;
        if (P.r_lds <= 16) launch_with_lds(b2s_kernel<1>, grid, slds, stream, P);
        else launch_with_lds(b2s_kernel<2>, grid, slds, stream, P);
    } else if (C2 == 256) {
        switch (rank_blocks(P.r_lds)) {
        case 1: launch_with_lds(b2_kernel<256, 1>, grid, lds, stream, P); break;
        case 2: launch_with_lds(b2_kernel<256, 2>, grid, lds, stream, P); break;
        case 4: launch_with_lds(b2_kernel<256, 4>, grid, lds, stream, P); break;
        default: launch_with_lds(b2_kernel<256, 8>, grid, lds, stream, P); break;
        }
    } else {
        launch_with_lds(b2_kernel<128, 16>, grid, lds, stream, P);
    }
    return finish_launch(slot, stream);
}

hipError_t launch_b2w(const void *X, const uint32_t *keep, const float *dS, int m, int k, int RS, int rows,
                      const AdapterSource &src, int items, float *part, const int32_t *ad_items, hipStream_t stream,
                      const uint16_t *dss, int dss_ld) {
    B2WParams P;
    P.X = (const uint16_t *)X;
    P.keep = keep;
    P.dS = dS;
    P.dss = dss;
    P.dss_ld = dss_ld;
    P.m = m;
    P.k = k;
    P.RS = RS;
    P.KW = (k + 31) / 32;
    P.work = make_work(src, kTabBwd);
    P.work.rows_per_chunk = rows;
    P.nct = cdiv(k, 256);
    P.part = part;
    const int mt = b2w_blocks(r_lds_of(src));
    // above 32 ranks the rank side comes split from B1's finishing launch
    if (mt >= 4 && (dss == nullptr || dss_ld < 32 * mt || (((uintptr_t)dss) & 15) != 0)) return hipErrorInvalidValue;
    (void)hipGetLastError();
    if (items > 0 && m > 0) {
        const dim3 grid((unsigned)items, (unsigned)P.nct);
        const int slot = prof_begin("b2_da", stream);
        switch (mt) {
        case 1: launch_with_lds(b2w_kernel<1>, grid, (size_t)B2W<1>::LDS, stream, P); break;
        case 2: launch_with_lds(b2w_kernel<2>, grid, (size_t)B2W<2>::LDS, stream, P); break;
        case 4: launch_with_lds(b2w_kernel<4>, grid, (size_t)B2W<4>::LDS, stream, P); break;
        default: launch_with_lds(b2w_kernel<8>, grid, (size_t)B2W<8>::LDS, stream, P); break;
        }
        const hipError_t e = finish_launch(slot, stream);
        if (e != hipSuccess) return e;
    }
    DAReduceParams R;
    R.part = part;
    R.k = k;
    R.nct = P.nct;
    R.RPT = 16 * mt;
    R.work = P.work;
    R.items = src.table ? items : (m > 0 ? items : 0);
    R.ad_items = ad_items;
    const int nad = src.table ? src.num_adapters : 1;
    const size_t f4 = (size_t)P.nct * 256 * R.RPT / 4;
    const int slot = prof_begin("reduce_da", stream);
    hipLaunchKernelGGL(da_reduce_kernel, dim3((unsigned)((f4 + 255) / 256), (unsigned)nad), dim3(256), 0, stream, R);
    return finish_launch(slot, stream);
}

static GradReduceParams grad_params(int which, const float *part, int m, int k, int n, int RS,
                                    const AdapterSource &src, int rows, int slots) {
    GradReduceParams P;
    P.part = part;
    P.which = which;
    P.m = m;
    P.k = k;
    P.n = n;
    P.RS = RS;
    P.work = make_work(src, which == 0 ? kTabB1 : kTabBwd);
    P.work.rows_per_chunk = rows;
    P.chunk_cap = slots;
    return P;
}

static int grad_gx(int which, int k, int n, int RS) {
    const size_t per = (size_t)(which == 0 ? n : k) * (size_t)RS;
    return (int)std::min<size_t>((per + 63) / 64, 8192);
}

hipError_t launch_grad_reduce(int which, const float *part, int m, int k, int n, int RS,
                              const AdapterSource &src, int rows, int slots, hipStream_t stream) {
    const GradReduceParams P = grad_params(which, part, m, k, n, RS, src, rows, slots);
    const int nad = src.table ? src.num_adapters : 1;
    const int gx = grad_gx(which, k, n, RS);
    (void)hipGetLastError();
    const int slot = prof_begin(which == 0 ? "reduce_db" : "reduce_da", stream);
    hipLaunchKernelGGL(grad_reduce_kernel, dim3(gx, nad), dim3(256), 0, stream, P);
    return finish_launch(slot, stream);
}

hipError_t launch_b1_reduce(const float *dSpart, int nparts, float *dS, const float *dBpart, int m, int n,
                            int RS, const AdapterSource &src, int rows, int slots, hipStream_t stream,
                            uint16_t *dss, int dss_ld) {
    B1FinishParams P;
    P.dspart = dSpart;
    P.nparts = nparts;
    P.ds = dS;
    P.dss = dss;
    P.dss_ld = dss_ld;
    P.m = m;
    P.n = n;
    P.RS = RS;
    P.dbpart = dBpart;
    P.work = make_work(src, kTabB1);
    P.work.rows_per_chunk = rows;
    P.groups = src.table ? slots : cdiv(m, rows);
    // one partial and no split rows: B1 wrote dS itself, nothing to do.
    // Otherwise about 4 elements per thread.
    const int W = dss ? std::max(RS, 128) : RS;
    P.ds_wpg = ((nparts > 1 || dss) && m > 0) ? std::max(1, cdiv((long)rows * W, 1024)) : 0;
    P.db_gx = std::max(1, cdiv((long)RS * n / 4, 256));
    const int nad = src.table ? src.num_adapters : 1;
    const size_t blocks = (size_t)P.groups * P.ds_wpg + (size_t)P.db_gx * nad;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7FFFFFFFu) return hipErrorInvalidValue;
    (void)hipGetLastError();
    const int slot = prof_begin("reduce_ds_db", stream);
    hipLaunchKernelGGL(b1_finish_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, P);
    return finish_launch(slot, stream);
}

hipError_t launch_mask(uint64_t seed, uint64_t offset, int m, int k, float p, uint32_t *bits,
                       hipStream_t stream) {
    const size_t words = (size_t)m * ((k + 31) / 32);
    if (words == 0) return hipSuccess;
    (void)hipGetLastError();
    const int slot = prof_begin("dropout_mask", stream);
    hipLaunchKernelGGL(mask_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream, seed,
                       offset, m, k, drop_threshold(p), bits);
    return finish_launch(slot, stream);
}

}  // namespace lora
