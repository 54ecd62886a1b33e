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

#include "device_common.hpp"
#include "launch.hpp"

namespace lora {

// ===========================================================================
// Router: chunk tables for the low-rank kernels (papers.chlience.com notes,
// section 5 "FusedMultiLoRA": tile-level routing by adapter id).  Each
// non-empty segment with a valid adapter is cut into runs of at most
// rows_f1 (resp. rows_bwd) rows; a single work-group scans the segments.
// ===========================================================================
__global__ __launch_bounds__(1024) void router_kernel(const int64_t *seg_off, const int32_t *seg_ad,
                                                     int nseg, int m, const lora_adapter *adapters,
                                                     int nad, int r_cap, ChunkEntry *t0, int32_t *c0,
                                                     int rows0, int cap0, ChunkEntry *t1,
                                                     int32_t *c1, int rows1, int cap1) {
    __shared__ int sc0[1024], sc1[1024];
    const int tid = threadIdx.x;
    int carry0 = 0, carry1 = 0;
    for (int base = 0; base < nseg; base += 1024) {
        const int s = base + tid;
        int lo = 0, hi = 0, a = -1, n0 = 0, n1 = 0;
        if (s < nseg) {
            const int64_t o0 = seg_off[s], o1 = seg_off[s + 1];
            lo = (int)max((int64_t)0, min(o0, (int64_t)m));
            hi = (int)max((int64_t)lo, min(o1, (int64_t)m));
            a = seg_ad[s];
            bool ok = a >= 0 && a < nad && hi > lo;
            if (ok) {
                const int r = adapters[a].r;
                ok = r >= 1 && r <= r_cap;
            }
            if (ok) {
                n0 = (hi - lo + rows0 - 1) / rows0;
                n1 = (hi - lo + rows1 - 1) / rows1;
            }
        }
        sc0[tid] = n0;
        sc1[tid] = n1;
        __syncthreads();
        for (int d = 1; d < 1024; d <<= 1) {
            const int v0 = tid >= d ? sc0[tid - d] : 0;
            const int v1 = tid >= d ? sc1[tid - d] : 0;
            __syncthreads();
            sc0[tid] += v0;
            sc1[tid] += v1;
            __syncthreads();
        }
        const int p0 = carry0 + sc0[tid] - n0;
        const int p1 = carry1 + sc1[tid] - n1;
        for (int q = 0; q < n0; ++q) {
            if (p0 + q < cap0) {
                ChunkEntry e;
                e.row_lo = lo + q * rows0;
                e.row_hi = min(hi, lo + (q + 1) * rows0);
                e.adapter = a;
                e.pad = 0;
                t0[p0 + q] = e;
            }
        }
        for (int q = 0; q < n1; ++q) {
            if (p1 + q < cap1) {
                ChunkEntry e;
                e.row_lo = lo + q * rows1;
                e.row_hi = min(hi, lo + (q + 1) * rows1);
                e.adapter = a;
                e.pad = 0;
                t1[p1 + q] = e;
            }
        }
        carry0 += sc0[1023];
        carry1 += sc1[1023];
        __syncthreads();
    }
    if (tid == 0) {
        c0[0] = min(carry0, cap0);
        c1[0] = min(carry1, cap1);
    }
}

static RowWork make_work(const AdapterSource &src, bool f1) {
    RowWork w;
    w.chunks = src.table ? (f1 ? src.chunks_f1 : src.chunks_bwd) : nullptr;
    w.chunk_count = src.table ? (f1 ? src.count_f1 : src.count_bwd) : nullptr;
    w.adapters = src.table;
    w.num_adapters = src.num_adapters;
    w.rows_per_chunk = f1 ? kF1Rows : kBwdRows;
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
// Work-group = 4 waves x 16 rows of one chunk, over one k-slice.  Lane l of a
// wave owns row (l % 16) and the 8 columns 8*(l/16).. of each 32-wide K step:
// exactly one Philox block and one MFMA A-fragment.  A is staged transposed
// in LDS (At[rr][kk]) per 128-column slice so its fragments are 16-B reads.
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
};

constexpr int kF1Ld = kF1KSub + 8;  // LDS row stride of At (elements)

template <int MAXT>
__global__ __launch_bounds__(256) void f1_kernel(F1Params P) {
    extern __shared__ uint4 f1_smem[];
    uint16_t *At = (uint16_t *)f1_smem;

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

    f32x4_t acc[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int k0 = kb; k0 < ke; k0 += kF1KSub) {
        __syncthreads();
        for (int idx = tid; idx < kF1KSub * rpad; idx += 256) {
            const int kk = idx / rpad, rr = idx - kk * rpad;
            uint16_t v = 0;
            if (rr < r && k0 + kk < ke) v = ad.A[(size_t)(k0 + kk) * r + rr];
            At[rr * kF1Ld + kk] = v;
        }
        __syncthreads();

        uint4 xv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c0 = k0 + 32 * t + 8 * g;
            xv[t] = (rvalid && c0 < ke) ? *(const uint4 *)(xrow + c0) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c0 = k0 + 32 * t + 8 * g;
            uint32_t byte = 0;
            if (rvalid && c0 < ke) byte = (T == 0) ? 0xFFu : keep_byte(ctr_row + (uint64_t)c0, P.seed, T);
            xv[t] = apply_keep(xv[t], byte);
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
                    const uint4 bf = *(const uint4 *)&At[(bt * 16 + li) * kF1Ld + 32 * t + 8 * g];
                    acc[bt] = mfma16x16x32(xv[t], bf, acc[bt]);
                }
            }
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

// ===========================================================================
// Fixed-order sum of split partials: out[i] = sum_p part[p*stride + i].
// ===========================================================================
__global__ __launch_bounds__(256) void sum_partials_kernel(const float *part, int nparts,
                                                           size_t stride, size_t count, float *out) {
    const size_t i4 = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i4 >= count) return;
    const bool vec = (stride & 3) == 0 && ((uintptr_t)out & 15) == 0 && ((uintptr_t)part & 15) == 0;
    if (i4 + 4 <= count && vec) {
        float4 a = *(const float4 *)(part + i4);
        for (int p = 1; p < nparts; ++p) {
            const float4 b = *(const float4 *)(part + (size_t)p * stride + i4);
            a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
        }
        *(float4 *)(out + i4) = a;
    } else {
        for (size_t i = i4; i < count && i < i4 + 4; ++i) {
            float a = part[i];
            for (int p = 1; p < nparts; ++p) a += part[(size_t)p * stride + i];
            out[i] = a;
        }
    }
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

    for (int rs = row_lo; rs < row_hi; rs += 64) {
        __syncthreads();
        for (int v = tid; v < 64 * (C1 / 8); v += 256) {
            const int rrow = v / (C1 / 8), cv = v - rrow * (C1 / 8);
            const int row = rs + rrow, col = n0 + cv * 8;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (row < row_hi && col < P.n) val = *(const uint4 *)(P.dY + (size_t)row * P.n + col);
            *(uint4 *)&Ys[rrow * LDY + cv * 8] = val;
        }
        for (int idx = tid; idx < 64 * rpad; idx += 256) {
            const int rrow = idx / rpad, rr = idx - rrow * rpad;
            const int row = rs + rrow;
            float v = 0.f;
            if (row < row_hi && rr < r) v = alpha * P.S[(size_t)row * P.RS + rr];
            Sts[rr * LDS_S + rrow] = v;
        }
        __syncthreads();

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

    for (int rs = row_lo; rs < row_hi; rs += 64) {
        __syncthreads();
        for (int blk = tid; blk < 8 * (C2 / 8); blk += 256) {
            const int rb = blk / (C2 / 8), cb = blk - rb * (C2 / 8);
            const int col = k0 + cb * 8;
            uint4 v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int row = rs + rb * 8 + e;
                uint4 x = make_uint4(0, 0, 0, 0);
                if (row < row_hi && col < P.k) {
                    x = *(const uint4 *)(P.X + (size_t)row * P.k + col);
                    if (P.keep != nullptr) {
                        const uint32_t word = P.keep[(size_t)row * P.KW + (col >> 5)];
                        x = apply_keep(x, (word >> (col & 31)) & 0xFFu);
                    }
                }
                v[e] = x;
            }
            uint4 o[8];
            transpose8x8(v, o);
#pragma unroll
            for (int c = 0; c < 8; ++c) *(uint4 *)&Xt[(cb * 8 + c) * LDX + rb * 8] = o[c];
        }
        for (int idx = tid; idx < 64 * rpad; idx += 256) {
            const int rrow = idx / rpad, rr = idx - rrow * rpad;
            const int row = rs + rrow;
            float v = 0.f;
            if (row < row_hi && rr < r) v = s * P.dS[(size_t)row * P.RS + rr];
            dSts[rr * LDS_S + rrow] = v;
        }
        __syncthreads();

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

__global__ __launch_bounds__(256) void grad_reduce_kernel(GradReduceParams P) {
    const int a = blockIdx.y;
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

    for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
        const size_t ro = e / cols_out, co = e - ro * cols_out;
        float acc = 0.f;
        for (int c = 0; c < nch; ++c) {
            if (P.work.chunks != nullptr) {
                const ChunkEntry ce = P.work.chunks[c];
                if (ce.adapter != a) continue;
            }
            acc += P.part[(size_t)c * chunk_stride + ro * row_stride + co];
        }
        outp[e] = (uint16_t)f32_to_bf16_rne(acc);
    }
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
                         int32_t *c_f1, int cap_f1, ChunkEntry *t_bwd, int32_t *c_bwd, int cap_bwd,
                         hipStream_t stream) {
    (void)hipGetLastError();
    const int slot = prof_begin("router", stream);
    hipLaunchKernelGGL(router_kernel, dim3(1), dim3(1024), 0, stream, seg_off, seg_adapter, nseg, m,
                       adapters, nad, r_cap, t_f1, c_f1, kF1Rows, cap_f1, t_bwd, c_bwd, kBwdRows,
                       cap_bwd);
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
static void launch_with_lds(Kernel kernel, dim3 grid, size_t lds, hipStream_t stream, const Params &P) {
    if (lds > 64 * 1024) (void)hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(kernel, grid, dim3(256), lds, stream, P);
}

static int r_lds_of(const AdapterSource &src) {
    const int rc = src.table ? src.r_cap : src.r;
    return ((rc + 15) / 16) * 16;
}

hipError_t launch_f1(const void *X, int m, int k, const AdapterSource &src, int chunk_cap,
                     uint64_t seed, uint64_t offset, uint32_t *keep_bits, float *out, int RS,
                     int KS, int ksl, hipStream_t stream) {
    F1Params P;
    P.X = (const uint16_t *)X;
    P.m = m;
    P.k = k;
    P.work = make_work(src, true);
    P.seed = seed;
    P.offset = offset;
    P.keep_bits = keep_bits;
    P.out = out;
    P.RS = RS;
    P.ksl = ksl;
    P.KW = (k + 31) / 32;
    P.r_lds = r_lds_of(src);
    const size_t lds = (size_t)P.r_lds * kF1Ld * sizeof(uint16_t);
    const dim3 grid(chunk_cap, KS);
    (void)hipGetLastError();
    const int slot = prof_begin("f1_mask_down", stream);
    switch (rank_blocks(P.r_lds)) {
    case 1: launch_with_lds(f1_kernel<1>, grid, lds, stream, P); break;
    case 2: launch_with_lds(f1_kernel<2>, grid, lds, stream, P); break;
    case 4: launch_with_lds(f1_kernel<4>, grid, lds, stream, P); break;
    case 8: launch_with_lds(f1_kernel<8>, grid, lds, stream, P); break;
    default: launch_with_lds(f1_kernel<16>, grid, lds, stream, P); break;
    }
    return finish_launch(slot, stream);
}

hipError_t launch_sum_partials(const float *part, int nparts, size_t part_stride, size_t count,
                               float *out, const char *name, hipStream_t stream) {
    if (count == 0) return hipSuccess;
    (void)hipGetLastError();
    const int slot = prof_begin(name, stream);
    const size_t blocks = (count + 1023) / 1024;
    hipLaunchKernelGGL(sum_partials_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part,
                       nparts, part_stride, count, out);
    return finish_launch(slot, stream);
}

size_t b1_lds_bytes(int C1, int r_lds) {
    return (size_t)r_lds * (C1 + 8) * 2 + (size_t)64 * (C1 + 8) * 2 + (size_t)r_lds * 68 * 4;
}
size_t b2_lds_bytes(int C2, int r_lds) { return (size_t)C2 * 72 * 2 + (size_t)r_lds * 68 * 4; }

hipError_t launch_b1(const void *dY, const float *S, int m, int n, int RS, const AdapterSource &src,
                     int chunk_cap, int C1, float *dSpart, float *dBpart, hipStream_t stream) {
    B1Params P;
    P.dY = (const uint16_t *)dY;
    P.S = S;
    P.m = m;
    P.n = n;
    P.RS = RS;
    P.work = make_work(src, false);
    P.dSpart = dSpart;
    P.dBpart = dBpart;
    P.r_lds = r_lds_of(src);
    const size_t lds = b1_lds_bytes(C1, P.r_lds);
    (void)hipGetLastError();
    const int slot = prof_begin("b1_ds_db", stream);
    const dim3 grid(chunk_cap, cdiv(n, C1));
    if (C1 == 256) {
        switch (rank_blocks(P.r_lds)) {
        case 1: launch_with_lds(b1_kernel<256, 1>, grid, lds, stream, P); break;
        case 2: launch_with_lds(b1_kernel<256, 2>, grid, lds, stream, P); break;
        case 4: launch_with_lds(b1_kernel<256, 4>, grid, lds, stream, P); break;
        default: launch_with_lds(b1_kernel<256, 8>, grid, lds, stream, P); break;
        }
    } else {
        launch_with_lds(b1_kernel<128, 16>, grid, lds, stream, P);
    }
    return finish_launch(slot, stream);
}

hipError_t launch_b2(const void *X, const uint32_t *keep, const float *dS, int m, int k, int RS,
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
    P.work = make_work(src, false);
    P.dApart = dApart;
    P.r_lds = r_lds_of(src);
    const size_t lds = b2_lds_bytes(C2, P.r_lds);
    (void)hipGetLastError();
    const int slot = prof_begin("b2_da", stream);
    const dim3 grid(chunk_cap, cdiv(k, C2));
    if (C2 == 256) {
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

hipError_t launch_grad_reduce(int which, const float *part, int m, int k, int n, int RS,
                              const AdapterSource &src, int chunk_cap, hipStream_t stream) {
    GradReduceParams P;
    P.part = part;
    P.which = which;
    P.m = m;
    P.k = k;
    P.n = n;
    P.RS = RS;
    P.work = make_work(src, false);
    P.chunk_cap = chunk_cap;
    const int nad = src.table ? src.num_adapters : 1;
    const size_t per = (size_t)(which == 0 ? n : k) * (size_t)RS;
    const int gx = (int)std::min<size_t>((per + 255) / 256, 4096);
    (void)hipGetLastError();
    const int slot = prof_begin(which == 0 ? "reduce_db" : "reduce_da", stream);
    hipLaunchKernelGGL(grad_reduce_kernel, dim3(gx, nad), dim3(256), 0, stream, P);
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
