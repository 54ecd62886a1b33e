// Device-side building blocks of the gfx950 LoRA path: bf16 bit helpers,
// MFMA wrappers, the dropout counter generator, and the parameter blocks the
// host launcher hands to the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_fused.h"

namespace lora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (raw 16-bit patterns)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even fp32 -> bf16 (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two fp32 values -> packed bf16 pair, round to nearest even (one gfx950
// v_cvt_pk_bf16_f32; agrees with f32_to_bf16_rne on finite inputs).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){lo, hi}, bf16x2_t));
}

// Split v into bf16 hi + lo with v ~= hi + lo to ~2^-17 relative (both halves
// rounded to nearest even; v - hi is exact in fp32).
__device__ __forceinline__ void split_bf16(float v, uint32_t &hi, uint32_t &lo) {
    hi = pack_bf16x2(v, 0.f) & 0xFFFFu;
    lo = pack_bf16x2(v - bf16_to_f32(hi), 0.f) & 0xFFFFu;
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return lo16 | (hi16 << 16); }


// ---------------------------------------------------------------------------
// MFMA: D = A*B + C with 8 bf16 per lane for each operand.
// 32x32x16: operand lane l holds row/column (l % 32) and K slots 8*(l/32)..+7;
//           result lane l, register v holds D[8*(v/4) + 4*(l/32) + v%4][l % 32].
// 16x16x32: operand lane l holds row/column (l % 16) and K slots 8*(l/16)..+7;
//           result lane l, register v holds D[4*(l/16) + v][l % 16].
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16_t mfma32x32x16(const uint4 &a, const uint4 &b, const f32x16_t &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4 &a, const uint4 &b, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                    __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// acc += a * b on the accumulator's own AGPRs.  The tied operand keeps each
// accumulator at a fixed register across a K loop (the builtin leaves the
// allocator free to rotate 256 accumulator registers every trip).  The
// compiler does not model the latency of this form: mfma_drain() must run
// before anything but another in-place MFMA touches the accumulators.
__device__ __forceinline__ void mfma16x16x32_inplace(f32x4_t &acc, const uint4 &a, const uint4 &b) {
    typedef int i32x4_t __attribute__((ext_vector_type(4)));
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                 : "+a"(acc)
                 : "v"(__builtin_bit_cast(i32x4_t, a)), "v"(__builtin_bit_cast(i32x4_t, b)));
}
// Wait states after the last in-place MFMA before its result is read by any
// other instruction (a 16x16x32 MFMA needs at most 11; this gives 32).
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 15\n\ts_nop 15" ::: "memory"); }
// Wait states between VALU writes of two source operands and the in-place
// MFMAs that read them (16; the compiler inserts none before inline asm).
// The operands pass through the asm so their producers stay above it.
__device__ __forceinline__ void mfma_src_ready(uint4 &a, uint4 &b) {
    typedef int i32x4_t __attribute__((ext_vector_type(4)));
    i32x4_t x = __builtin_bit_cast(i32x4_t, a), y = __builtin_bit_cast(i32x4_t, b);
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
    a = __builtin_bit_cast(uint4, x);
    b = __builtin_bit_cast(uint4, y);
}
__device__ __forceinline__ void mfma_src_ready(uint4 &a) {
    typedef int i32x4_t __attribute__((ext_vector_type(4)));
    i32x4_t x = __builtin_bit_cast(i32x4_t, a);
    asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x));
    a = __builtin_bit_cast(uint4, x);
}

// Eight fp32 values -> hi and lo bf16 fragments.
__device__ __forceinline__ void split_frag(const float v[8], uint4 &hi, uint4 &lo) {
    // pairs through v_cvt_pk_bf16_f32: the hi pair, each element's residual
    // against its hi half, the lo pair (the same bits as split_bf16 per element)
    uint32_t h[4], l[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        h[p] = pack_bf16x2(v[2 * p], v[2 * p + 1]);
        const float r0 = v[2 * p] - __uint_as_float(h[p] << 16);
        const float r1 = v[2 * p + 1] - __uint_as_float(h[p] & 0xFFFF0000u);
        l[p] = pack_bf16x2(r0, r1);
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// One half of split_frag chosen per lane: the hi parts, or (want_lo) the lo
// parts, of the same 8 values (bit-identical to split_frag's output).
__device__ __forceinline__ uint4 split_frag_half(const float v[8], bool want_lo) {
    float d[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = v[e] - (want_lo ? bf16_to_f32(f32_to_bf16_rne(v[e])) : 0.f);
    return make_uint4(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]), pack_bf16x2(d[4], d[5]),
                      pack_bf16x2(d[6], d[7]));
}

// 8x8 bf16 transpose held in one thread: in[e] is row e (8 elements, 16 B);
// out[c] becomes column c (rows 0..7).  v_perm picks the 16-bit halves.
__device__ __forceinline__ void transpose8x8(const uint4 in[8], uint4 out[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 &r0 = in[2 * q];
            const uint4 &r1 = in[2 * q + 1];
            uint32_t a0 = (c >> 1) == 0 ? r0.x : (c >> 1) == 1 ? r0.y : (c >> 1) == 2 ? r0.z : r0.w;
            uint32_t a1 = (c >> 1) == 0 ? r1.x : (c >> 1) == 1 ? r1.y : (c >> 1) == 2 ? r1.z : r1.w;
            w[q] = __builtin_amdgcn_perm(a1, a0, sel);
        }
        out[c] = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// ---------------------------------------------------------------------------
// Dropout counter generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
// SC'11).  Each round multiplies words 0 and 2 by two fixed odd constants,
// keeps both halves of the products and mixes the high halves with words 1
// and 3 and the round key; the key advances by two Weyl increments between
// rounds.  Counter words 2 and 3 are always zero here.
// ---------------------------------------------------------------------------
struct PhiloxOut {
    uint32_t w[4];
};

// a ^ b ^ k in one instruction (gfx950 three-input bit operation, truth
// table 0x96); k is wave-uniform.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t k) {
    uint32_t d;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(d) : "v"(a), "v"(b), "s"(k));
    return d;
}

__device__ __forceinline__ PhiloxOut philox10(uint64_t block, uint64_t seed) {
    constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    // round 1 on (b_lo, b_hi, 0, 0): the word-2 product is zero
    const uint64_t q0 = (uint64_t)(uint32_t)block * M0;
    uint32_t c0 = (uint32_t)(block >> 32) ^ k0;
    uint32_t c1 = 0u;
    uint32_t c2 = (uint32_t)(q0 >> 32) ^ k1;
    uint32_t c3 = (uint32_t)q0;
    k0 += W0;
    k1 += W1;
    // round 2: word 1 is zero
    {
        const uint64_t p0 = (uint64_t)c0 * M0;
        const uint64_t p1 = (uint64_t)c2 * M1;
        c0 = (uint32_t)(p1 >> 32) ^ k0;
        c2 = xor3((uint32_t)(p0 >> 32), c3, k1);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        k0 += W0;
        k1 += W1;
    }
#pragma unroll
    for (int rnd = 2; rnd < 10; ++rnd) {
        // one 32x32->64 multiply gives both halves of each product
        const uint64_t p0 = (uint64_t)c0 * M0;
        const uint64_t p1 = (uint64_t)c2 * M1;
        c0 = xor3((uint32_t)(p1 >> 32), c1, k0);
        c2 = xor3((uint32_t)(p0 >> 32), c3, k1);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        k0 += W0;
        k1 += W1;
    }
    PhiloxOut o;
    o.w[0] = c0; o.w[1] = c1; o.w[2] = c2; o.w[3] = c3;
    return o;
}

// Keep bits of the 8 elements with counters c8 .. c8+7 (c8 % 8 == 0): bit e
// set iff uniform e >= T.  Uniform e is 16-bit half (e & 1) of word e >> 1.
__device__ __forceinline__ uint32_t keep_byte(uint64_t c8, uint64_t seed, uint32_t T) {
    const PhiloxOut o = philox10(c8 >> 3, seed);
    uint32_t b = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        b |= ((o.w[q] & 0xFFFFu) >= T ? 1u : 0u) << (2 * q);
        b |= ((o.w[q] >> 16) >= T ? 1u : 0u) << (2 * q + 1);
    }
    return b;
}

// Zero the bf16 elements of an 8-element fragment whose keep bit is clear.
__device__ __forceinline__ uint4 apply_keep(uint4 v, uint32_t byte) {
    uint32_t m[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        m[q] = ((byte >> (2 * q)) & 1u ? 0x0000FFFFu : 0u) | ((byte >> (2 * q + 1)) & 1u ? 0xFFFF0000u : 0u);
    return make_uint4(v.x & m[0], v.y & m[1], v.z & m[2], v.w & m[3]);
}

// Keep test and masking of 8 bf16 elements in packed 16-bit arithmetic.
// tm1x2 holds T - 1 in both halves (T >= 1).  For each 16-bit uniform u,
// saturating u - (T - 1) is nonzero iff u >= T; its minimum with 1 is the
// keep bit, and multiplying the bf16 bit pattern by it keeps or zeroes the
// element.  Returns the keep byte (bit e for element e) and the masked x.
__device__ __forceinline__ uint32_t pk_sub_sat_u16(uint32_t a, uint32_t b) {
    uint32_t d;
    asm("v_pk_sub_u16 %0, %1, %2 clamp" : "=v"(d) : "v"(a), "s"(b));
    return d;
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    uint32_t d;
    asm("v_pk_min_u16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ uint32_t pk_mul_lo_u16(uint32_t a, uint32_t b) {
    uint32_t d;
    asm("v_pk_mul_lo_u16 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ uint32_t keep_and_mask(const PhiloxOut &o, uint32_t tm1x2, const uint4 &x,
                                                  uint4 &xm) {
    const uint32_t one2 = 0x00010001u;
    uint32_t kq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) kq[q] = pk_min_u16(pk_sub_sat_u16(o.w[q], tm1x2), one2);
    xm = make_uint4(pk_mul_lo_u16(x.x, kq[0]), pk_mul_lo_u16(x.y, kq[1]), pk_mul_lo_u16(x.z, kq[2]),
                    pk_mul_lo_u16(x.w, kq[3]));
    // low-half bits land on 0,2,4,6 and high-half bits on 16,18,20,22
    const uint32_t t = kq[0] | (kq[1] << 2) | (kq[2] << 4) | (kq[3] << 6);
    return (t & 0x55u) | ((t >> 15) & 0xAAu);
}

// Dropout threshold and inverted-dropout scale from p (identical arithmetic on
// every device and the host: T in double, exact for float p in [0, 1)).
__host__ __device__ __forceinline__ uint32_t drop_threshold(float p) {
    return (uint32_t)((double)p * 65536.0 + 0.5);
}
__host__ __device__ __forceinline__ float drop_scale(float p) { return 1.0f / (1.0f - p); }

// Buffer resource over `bytes` bytes from `base`; loads past the end return 0
// and stores past the end are dropped, so edge tiles need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint64_t bytes) {
    const uint32_t nrec = (uint32_t)(bytes < 0x7FFFFFF0ull ? bytes : 0x7FFFFFF0ull);
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)nrec, 0x00020000);
}
constexpr uint32_t kOOB = 0x80000000u;  // an offset beyond every resource

// ---------------------------------------------------------------------------
// Direct-to-LDS loads and LDS transposing reads (gfx950)
// ---------------------------------------------------------------------------
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// s_waitcnt with only the vector-memory counter constrained (vmcnt in bits
// 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Raw buffer descriptor words (base, stride 0, num_records, gfx9 dword3).
typedef int sgpr4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ sgpr4_t make_desc(const void *base, uint32_t bytes) {
    const uint64_t b = (uint64_t)base;
    return sgpr4_t{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}
// 16-byte direct-to-LDS load: lane l's 16 bytes from desc+voff land at LDS
// byte lds_base + 16*l.  Issued as inline asm so the compiler's wait-count
// insertion does not serialise later LDS reads behind it; completion is
// tracked by the explicit vmcnt waits of the K loop.
// M0 is saved and restored around the load.
__device__ __forceinline__ void dma16(sgpr4_t desc, uint32_t voff, uint32_t lds_base) {
    uint32_t saved_m0;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved_m0)
        : "v"(voff), "s"(desc), "s"(lds_base)
        : "memory");
}

// Transposing LDS read of 4 bf16 (8 bytes): within each 16-lane group, lane
// l receives element (l % 4) of the 8-byte rows addressed by lanes
// 4*i + l/4, i = 0..3 -- i.e. given 4 rows x 16 columns addressed as 4-column
// pieces, every lane gets one column's 4 consecutive rows.
__device__ __forceinline__ uint2 lds_read_tr4(const lds_char *p) {
    const v4s_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t *)p);
    return __builtin_bit_cast(uint2, v);
}

// Tiles of 256 bf16 columns have 512-byte LDS rows with an XOR swizzle of
// their 16-byte chunks that is conflict-free both for 16-lane b128 reads of
// 16 consecutive rows and for 32-lane transposing reads of rows {0-3, 8-11}
// (or {4-7, 12-15}) over two chunks.  The transposing reads hand each lane 8
// consecutive rows of one column: the MFMA operand of a contraction over rows.
__device__ __forceinline__ int swz512(int r) {
    return ((r & 3) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 3);
}
__device__ __forceinline__ uint32_t swz512_off(int row, int chunk) {
    return (uint32_t)(row * 512 + ((chunk ^ swz512(row)) << 4));
}
// 8 consecutive rows (row0 .. row0+7, row0 % 8 == 0) of column 16*cb + (lane % 16)
// of a swizzled 512-byte-row tile, as one MFMA operand.
__device__ __forceinline__ uint4 tile_rows8(const lds_char *tile, int row0, int cb, int lane) {
    const int a = lane & 15;
    const int chunk = 2 * cb + ((a & 3) >> 1);
    const int row = row0 + (a >> 2);
    const uint2 lo = lds_read_tr4(tile + swz512_off(row, chunk) + (a & 1) * 8);
    const uint2 hi = lds_read_tr4(tile + swz512_off(row + 4, chunk) + (a & 1) * 8);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}
constexpr uint32_t kOOBL = 0x80000000u;  // an offset beyond every descriptor range

// ---------------------------------------------------------------------------
// Work items of the low-rank kernels: a run of rows inside one segment.
// ---------------------------------------------------------------------------
struct ChunkEntry {
    int32_t row_lo;
    int32_t row_hi;
    int32_t adapter;
    int32_t pad;
};

struct AdapterView {
    const uint16_t *A;  // k x r
    const uint16_t *B;  // r x n
    uint16_t *dA;
    uint16_t *dB;
    int32_t r;
    float alpha;
    float p;
};

__device__ __forceinline__ AdapterView load_adapter(const lora_adapter *tab, int a) {
    const lora_adapter e = tab[a];
    AdapterView v;
    v.A = (const uint16_t *)e.A;
    v.B = (const uint16_t *)e.B;
    v.dA = (uint16_t *)e.dA;
    v.dB = (uint16_t *)e.dB;
    v.r = e.r;
    v.alpha = e.alpha;
    v.p = e.p;
    return v;
}

// Where a kernel finds its rows and adapter: either one adapter over all rows
// (chunk c = rows [c*rows_per_chunk, ...)), or a device chunk table built by
// the router from the segment table.
struct RowWork {
    const ChunkEntry *chunks;  // NULL: single adapter
    const int32_t *chunk_count;
    const lora_adapter *adapters;
    int32_t num_adapters;
    int32_t rows_per_chunk;
    int32_t r_cap;             // ranks above this are treated as invalid (r_max)
    AdapterView single;
};

// Returns false if this chunk index has no work.
__device__ __forceinline__ bool resolve_chunk(const RowWork &w, int chunk, int m, int &row_lo,
                                              int &row_hi, AdapterView &ad) {
    if (w.chunks == nullptr) {
        row_lo = chunk * w.rows_per_chunk;
        if (row_lo >= m) return false;
        row_hi = min(m, row_lo + w.rows_per_chunk);
        ad = w.single;
        return true;
    }
    if (chunk >= w.chunk_count[0]) return false;
    const ChunkEntry e = w.chunks[chunk];
    row_lo = e.row_lo;
    row_hi = e.row_hi;
    ad = load_adapter(w.adapters, e.adapter);
    if (ad.r < 1 || ad.r > w.r_cap) return false;
    return row_hi > row_lo;
}

}  // namespace lora
