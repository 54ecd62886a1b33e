// Host side of mixed-adapter batching: the greedy token-capacity packer that
// turns a global batch's samples into microbatches, the segment table of one
// microbatch (the input of the mixed-adapter entry points), and the check of
// the pipeline dependency between an adapter's consecutive global batches.
//
// Packing (papers.chlience.com notes on LoRAFusion, section 4 "Multi-LoRA
// scheduler"; juhe.plus blog, section 4.2 step 2): microbatches hold at most
// `capacity` tokens.  The pages' scheduler solves a two-stage MILP and falls
// back to a greedy packing when the solver times out; this is that greedy
// part, read as first-fit decreasing.  First fit runs on a max-tree over the
// microbatches' free tokens, so placing a sample costs O(log #microbatches).
//
// Bubble lemma (same sections, step 1): with S pipeline stages, if a sample
// of adapter a's global batch j is in microbatch k, no sample of a's next
// global batch may be in a microbatch before k + S - 1.
#include <algorithm>
#include <cstdint>
#include <numeric>
#include <tuple>
#include <vector>

#include "host_status.hpp"
#include "lora_fused.h"

namespace {

// Max-tree over the free tokens of microbatches 0 .. leaves-1 (leaves not yet
// opened hold -1, below any request): find() returns the lowest index whose
// free tokens cover the request, or -1.
class FirstFitTree {
  public:
    explicit FirstFitTree(int leaves) {
        while (size_ < leaves) size_ <<= 1;
        t_.assign(2 * (size_t)size_, -1);
    }
    void set(int i, int64_t v) {
        size_t x = (size_t)i + size_;
        t_[x] = v;
        for (x >>= 1; x >= 1; x >>= 1) t_[x] = std::max(t_[2 * x], t_[2 * x + 1]);
    }
    int64_t get(int i) const { return t_[(size_t)i + size_]; }
    int find(int64_t need) const {
        if (t_[1] < need) return -1;
        size_t x = 1;
        while (x < (size_t)size_) x = t_[2 * x] >= need ? 2 * x : 2 * x + 1;
        return (int)(x - size_);
    }

  private:
    int size_ = 1;
    std::vector<int64_t> t_;
};

}  // namespace

extern "C" lora_status lora_pack_greedy(const int32_t *lengths, int32_t num_samples, int64_t capacity,
                                        int32_t *mb_of_sample, int32_t *num_microbatches) {
    using namespace lora;
    if (num_microbatches == nullptr) return host_fail(LORA_ERR_INVALID_ARG, "num_microbatches is NULL");
    if (num_samples < 0) return host_fail(LORA_ERR_INVALID_ARG, "num_samples = %d is negative", num_samples);
    if (capacity < 1) return host_fail(LORA_ERR_INVALID_ARG, "capacity = %lld must be >= 1", (long long)capacity);
    if (num_samples > 0 && (lengths == nullptr || mb_of_sample == nullptr))
        return host_fail(LORA_ERR_INVALID_ARG, "NULL host array");
    for (int32_t i = 0; i < num_samples; ++i)
        if (lengths[i] < 1 || lengths[i] > capacity)
            return host_fail(LORA_ERR_INVALID_ARG, "sample %d has length %d outside [1, capacity = %lld]", i,
                             lengths[i], (long long)capacity);
    std::vector<int32_t> order(num_samples);
    std::iota(order.begin(), order.end(), 0);
    // longest first; the stable sort keeps equal lengths in sample order
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return lengths[a] > lengths[b]; });
    FirstFitTree tree(std::max(num_samples, 1));
    int32_t opened = 0;
    for (int32_t i : order) {
        int b = tree.find(lengths[i]);
        if (b < 0) {
            b = opened++;
            tree.set(b, capacity - lengths[i]);
        } else {
            tree.set(b, tree.get(b) - lengths[i]);
        }
        mb_of_sample[i] = b;
    }
    *num_microbatches = opened;
    return LORA_OK;
}

extern "C" lora_status lora_microbatch_segments(const int32_t *lengths, const int32_t *adapter_of_sample,
                                                const int32_t *mb_of_sample, int32_t num_samples,
                                                int32_t num_adapters, int32_t mb, int32_t *sample_order,
                                                int32_t *num_members, int64_t *seg_off, int32_t *seg_adapter,
                                                int32_t *num_segments) {
    using namespace lora;
    if (num_members == nullptr || num_segments == nullptr || seg_off == nullptr)
        return host_fail(LORA_ERR_INVALID_ARG, "NULL output");
    if (num_samples < 0 || num_adapters < 1)
        return host_fail(LORA_ERR_INVALID_ARG, "num_samples = %d, num_adapters = %d", num_samples, num_adapters);
    if (num_samples > 0 &&
        (lengths == nullptr || adapter_of_sample == nullptr || mb_of_sample == nullptr || sample_order == nullptr ||
         seg_adapter == nullptr))
        return host_fail(LORA_ERR_INVALID_ARG, "NULL host array");
    // members bucketed by adapter (counting sort: sample order within a bucket)
    std::vector<int32_t> count(num_adapters + 1, 0);
    for (int32_t i = 0; i < num_samples; ++i) {
        if (mb_of_sample[i] != mb) continue;
        const int32_t a = adapter_of_sample[i];
        if (a < 0 || a >= num_adapters)
            return host_fail(LORA_ERR_INVALID_ARG, "sample %d uses adapter %d outside [0, %d)", i, a, num_adapters);
        if (lengths[i] < 1) return host_fail(LORA_ERR_INVALID_ARG, "sample %d has length %d", i, lengths[i]);
        ++count[a + 1];
    }
    for (int32_t a = 0; a < num_adapters; ++a) count[a + 1] += count[a];
    const int32_t members = count[num_adapters];
    std::vector<int32_t> pos(count.begin(), count.end() - 1);
    for (int32_t i = 0; i < num_samples; ++i)
        if (mb_of_sample[i] == mb) sample_order[pos[adapter_of_sample[i]]++] = i;
    // one segment per adapter present
    int32_t ns = 0;
    int64_t rows = 0;
    seg_off[0] = 0;
    for (int32_t a = 0; a < num_adapters; ++a) {
        if (count[a + 1] == count[a]) continue;
        for (int32_t q = count[a]; q < count[a + 1]; ++q) rows += lengths[sample_order[q]];
        seg_adapter[ns] = a;
        seg_off[++ns] = rows;
    }
    *num_members = members;
    *num_segments = ns;
    return LORA_OK;
}

extern "C" lora_status lora_check_bubble_lemma(const int32_t *mb_of_sample, const int32_t *adapter_of_sample,
                                               const int32_t *batch_of_sample, int32_t num_samples,
                                               int32_t num_adapters, int32_t stages, int64_t *violations) {
    using namespace lora;
    if (violations == nullptr) return host_fail(LORA_ERR_INVALID_ARG, "violations is NULL");
    if (num_samples < 0 || num_adapters < 1 || stages < 1)
        return host_fail(LORA_ERR_INVALID_ARG, "num_samples = %d, num_adapters = %d, stages = %d", num_samples,
                         num_adapters, stages);
    if (num_samples > 0 && (mb_of_sample == nullptr || adapter_of_sample == nullptr || batch_of_sample == nullptr))
        return host_fail(LORA_ERR_INVALID_ARG, "NULL host array");
    // (adapter, batch, microbatch) of every sample, sorted: each (adapter,
    // batch) run then spans its earliest .. latest microbatch
    std::vector<std::tuple<int32_t, int32_t, int32_t>> v;
    v.reserve(num_samples);
    for (int32_t i = 0; i < num_samples; ++i) {
        const int32_t a = adapter_of_sample[i];
        if (a < 0 || a >= num_adapters)
            return host_fail(LORA_ERR_INVALID_ARG, "sample %d uses adapter %d outside [0, %d)", i, a, num_adapters);
        if (batch_of_sample[i] < 0 || mb_of_sample[i] < 0)
            return host_fail(LORA_ERR_INVALID_ARG, "sample %d has a negative batch or microbatch index", i);
        v.emplace_back(a, batch_of_sample[i], mb_of_sample[i]);
    }
    std::sort(v.begin(), v.end());
    int64_t bad = 0;
    int32_t prev_a = -1, prev_last = 0;  // adapter and latest microbatch of the previous run
    for (size_t s = 0; s < v.size();) {
        size_t e = s;
        while (e < v.size() && std::get<0>(v[e]) == std::get<0>(v[s]) && std::get<1>(v[e]) == std::get<1>(v[s])) ++e;
        const int32_t a = std::get<0>(v[s]), first = std::get<2>(v[s]), last = std::get<2>(v[e - 1]);
        if (a == prev_a && (int64_t)first < (int64_t)prev_last + stages - 1) ++bad;
        prev_a = a;
        prev_last = last;
        s = e;
    }
    *violations = bad;
    return LORA_OK;
}
