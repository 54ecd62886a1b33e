// Internal interface between the C-ABI layer (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lora_fused.h"

namespace lora {

struct ChunkEntry;

// Rows handled by one work item of each low-rank kernel.
constexpr int kF1Rows = 64;    // mask + down-projection
constexpr int kBwdRows = 256;  // dS/dB and dA kernels
constexpr int kF1KSub = 128;   // k columns per staged slice of A in F1

// F1's streaming form (each work-group covers all of k, no partial sums)
// serves ranks up to 32; its 32-bit buffer offsets need 64*k < 2^31.
inline bool f1_streaming(int r_lds, int64_t k) { return r_lds <= 32 && k * 64 < (int64_t(1) << 31); }

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
};

hipError_t launch_router(const int64_t *seg_off, const int32_t *seg_adapter, int nseg, int m,
                         const lora_adapter *adapters, int nad, int r_cap, ChunkEntry *t_f1,
                         int32_t *c_f1, int cap_f1, ChunkEntry *t_bwd, int32_t *c_bwd, int cap_bwd,
                         hipStream_t stream);

hipError_t launch_f1(const void *X, int m, int k, const AdapterSource &src, int chunk_cap,
                     uint64_t seed, uint64_t offset, uint32_t *keep_bits, float *out, int RS,
                     int KS, int ksl, hipStream_t stream);

hipError_t launch_sum_partials(const float *part, int nparts, size_t part_stride, size_t count,
                               float *out, const char *name, hipStream_t stream);

hipError_t launch_b1(const void *dY, const float *S, int m, int n, int RS, const AdapterSource &src,
                     int chunk_cap, int C1, float *dSpart, float *dBpart, hipStream_t stream);

hipError_t launch_b2(const void *X, const uint32_t *keep, const float *dS, int m, int k, int RS,
                     const AdapterSource &src, int chunk_cap, int C2, float *dApart,
                     hipStream_t stream);

// which = 0: dB (r x n per adapter from [chunk][RS][n]); 1: dA (k x r from [chunk][k][RS]).
hipError_t launch_grad_reduce(int which, const float *part, int m, int k, int n, int RS,
                              const AdapterSource &src, int chunk_cap, hipStream_t stream);

hipError_t launch_mask(uint64_t seed, uint64_t offset, int m, int k, float p, uint32_t *bits,
                       hipStream_t stream);

// GEMM: C = Arow * op(Bcol) (+ LoRA term).  nn: Bcol is K x N (W of the
// forward); otherwise Bcol is N x K (W seen transposed by the backward).
// epi 0: none; 1: + alpha*S*B (F2); 2: + s*keep.(dS A^T) (B3).
hipError_t launch_gemm(bool nn, int epi, const void *Arow, const void *Bcol, void *C, int M, int N,
                       int K, const float *Sx, int RS, const uint32_t *keep, int KW,
                       const AdapterSource &src, hipStream_t stream);

size_t gemm_lds_bytes();

}  // namespace lora
