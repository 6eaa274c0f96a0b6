// Cold pool -> hot pool block gather (zhichai.net explainer of "FlashMemory-DeepSeek-V4", section 2
// step 3: the selected blocks are moved from the CPU cold pool to the GPU; step 5: the loaded set is
// refreshed).
//
// Host: per request, diff the new ascending selection against the resident set, free the slots of
// blocks that left, give free slots to blocks that entered, and write the copy list and the new
// block table into the caller's pinned staging buffer.  Device: one kernel copies every entering
// 64-token block (one contiguous block-format record) from the cold pool into its slot, for every
// layer the selection serves, and copies the tables, for every request of the call.  A cold pool may be pinned host memory (the kernel
// reads it over the host link, zero-copy) or device memory.
#include <emmintrin.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <cstring>
#include <utility>
#include <vector>

#include "lsa_internal.hpp"

namespace lsa {

// Device-visible address of a buffer that is either device memory or pinned host memory.
lsa_status device_view(const void* ptr, const char* fn, const char* what, const void** out, bool* is_host) {
    hipPointerAttribute_t attr{};
    hipError_t e = hipPointerGetAttributes(&attr, ptr);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(LSA_ERR_INVALID, "%s: %s is neither device nor pinned host memory", fn, what);
    }
    if (attr.type == hipMemoryTypeDevice) {
        *out = ptr;
        *is_host = false;
        return LSA_OK;
    }
    if (attr.type == hipMemoryTypeHost) {
        void* dptr = nullptr;
        e = hipHostGetDevicePointer(&dptr, const_cast<void*>(ptr), 0);
        if (e != hipSuccess || dptr == nullptr) {
            (void)hipGetLastError();
            return fail(LSA_ERR_INVALID, "%s: %s is host memory that is not mapped for the device", fn, what);
        }
        *out = dptr;
        *is_host = true;
        return LSA_OK;
    }
    return fail(LSA_ERR_INVALID, "%s: %s has memory type %d (need device or pinned host)", fn, what,
                (int)attr.type);
}

namespace {

constexpr int kMaxBatch = 16;  // requests per copy-kernel launch

struct GatherJob {
    const char* cold;
    char* hot;
    const int* copies;  // (source block, slot) pairs, device-visible
    const int* tsrc;    // table pairs, device-visible
    int* tdst;
    long long cold_layer_bytes, hot_layer_bytes;
    int n_copies;       // per layer
};

struct GatherParams {
    int n_jobs;
    int block_bytes;
    int copy_off[kMaxBatch + 1];   // prefix of the jobs' copy counts (copies x layers)
    int table_off[kMaxBatch + 1];  // prefix of the jobs' table lengths (pairs)
    GatherJob job[kMaxBatch];
};

// Blocks are copied once per refresh: non-temporal 16-byte loads and stores.  With ordinary stores
// the L2 sent every written line to memory about twice (12.3M 64-byte write requests for 421 MB of
// blocks; 6.6M with these), and the copy took 88 us instead of 67 us.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4* q) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt(uint4* q, uint4 v) {
    const u32x4 t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(q));
}

// Copy c of the launch (jobs' copies concatenated) goes to group c, c + G, ...: one 64-token block
// at a time, 256 threads x 16-byte vectors, every load of the block in flight before its stores.
// The tables are copied with one grid-wide stride.  (One block per group with many groups measured
// faster than fewer groups that copy several blocks each.)
template <int PER>  // 16-byte vectors per thread per block (block_bytes / 4096)
__global__ __launch_bounds__(256) void gather_kernel(GatherParams p) {
    const int G = gridDim.x;
    const int n_table = p.table_off[p.n_jobs];
    for (int e = blockIdx.x * 256 + threadIdx.x; e < 2 * n_table; e += G * 256) {
        int j = 0;
        while (j + 1 < p.n_jobs && 2 * p.table_off[j + 1] <= e) ++j;
        const int k = e - 2 * p.table_off[j];
        p.job[j].tdst[k] = p.job[j].tsrc[k];
    }
    constexpr int STEP = PER > 8 ? 8 : PER;
    const int n_copies = p.copy_off[p.n_jobs];
    for (int c = blockIdx.x; c < n_copies; c += G) {
        int j = 0;
        while (j + 1 < p.n_jobs && p.copy_off[j + 1] <= c) ++j;
        const GatherJob& jb = p.job[j];
        const int kl = c - p.copy_off[j];
        const int layer = kl / jb.n_copies;
        const int k = kl - layer * jb.n_copies;
        const uint4* src = reinterpret_cast<const uint4*>(jb.cold + layer * jb.cold_layer_bytes +
                                                          (size_t)jb.copies[2 * k] * p.block_bytes);
        uint4* dst = reinterpret_cast<uint4*>(jb.hot + layer * jb.hot_layer_bytes + (size_t)jb.copies[2 * k + 1] * p.block_bytes);
#pragma unroll
        for (int v0 = 0; v0 < PER; v0 += STEP) {
            uint4 b[STEP];
#pragma unroll
            for (int v = 0; v < STEP; ++v) b[v] = load_nt(src + (v0 + v) * 256 + threadIdx.x);
#pragma unroll
            for (int v = 0; v < STEP; ++v) store_nt(dst + (v0 + v) * 256 + threadIdx.x, b[v]);
        }
    }
}


// Everything one request's gather decides before any state changes.
struct GatherPlan {
    std::vector<int> leave, enter, new_slot;
    std::vector<int> freestack;  // slots of the blocks that left, ascending block id
    std::vector<int> stage_buf;
    int kept = 0;
    const void* cold_dev = nullptr;
    const void* stage_dev = nullptr;
};

// Validate one request's arguments and plan its gather; fills the request's staging buffer (copy
// list, then table).  Touches no caller state.
lsa_status plan_gather(const lsa_gather_args* a, GatherPlan* P) {
    LSA_CHECK_ARG(a != nullptr, "lsa_gather_blocks: null args");
    LSA_CHECK_ARG(a->n_layers >= 0 && a->n_layers <= 256, "lsa_gather_blocks: n_layers=%d outside 0..256", a->n_layers);
    if (a->n_layers > 1) {
        LSA_CHECK_ARG(a->cold_layer_bytes >= a->n_blocks * (long long)a->block_bytes && a->cold_layer_bytes % 16 == 0,
                      "lsa_gather_blocks: cold_layer_bytes=%lld (>= n_blocks*block_bytes, multiple of 16)",
                      (long long)a->cold_layer_bytes);
        LSA_CHECK_ARG(a->hot_layer_bytes >= (long long)a->n_slots_total * a->block_bytes && a->hot_layer_bytes % 16 == 0,
                      "lsa_gather_blocks: hot_layer_bytes=%lld (>= n_slots_total*block_bytes, multiple of 16)",
                      (long long)a->hot_layer_bytes);
    }
    LSA_CHECK_ARG(a->n_blocks >= 1 && a->n_blocks <= (1ll << 30), "lsa_gather_blocks: n_blocks=%lld", (long long)a->n_blocks);
    LSA_CHECK_SUP(a->block_bytes == 16384 || a->block_bytes == 32768 || a->block_bytes == 65536,
                  "lsa_gather_blocks: block_bytes=%d (16, 32 or 64 KiB: the block format's sizes)", a->block_bytes);
    LSA_CHECK_ARG(a->n_new >= 0 && (a->n_new == 0 || a->new_ids), "lsa_gather_blocks: n_new=%d / new_ids", a->n_new);
    LSA_CHECK_ARG(a->slot_of_block && a->free_slots && a->n_free && a->n_copied && a->n_kept,
                  "lsa_gather_blocks: null host state pointer");
    LSA_CHECK_ARG(a->capacity >= 0 && a->n_slots_total >= a->capacity, "lsa_gather_blocks: capacity=%d n_slots_total=%d",
                  a->capacity, a->n_slots_total);
    LSA_CHECK_ARG(*a->n_free >= 0 && *a->n_free <= a->capacity, "lsa_gather_blocks: n_free=%d outside 0..capacity",
                  *a->n_free);
    LSA_CHECK_ARG(a->cold && a->hot && a->table_dev && a->stage, "lsa_gather_blocks: null buffer");
    for (int k = 0; k < a->n_new; ++k) {
        LSA_CHECK_ARG(a->new_ids[k] >= 0 && a->new_ids[k] < a->n_blocks, "lsa_gather_blocks: new_ids[%d]=%d out of range",
                      k, a->new_ids[k]);
        LSA_CHECK_ARG(k == 0 || a->new_ids[k] > a->new_ids[k - 1], "lsa_gather_blocks: new_ids not strictly ascending at %d", k);
    }
    if (a->n_new > a->capacity)
        return fail(LSA_ERR_CAPACITY, "lsa_gather_blocks: %d selected blocks exceed the %d hot slots", a->n_new, a->capacity);
    LSA_CHECK_ARG(a->stage_ints >= 4 * a->n_new, "lsa_gather_blocks: stage holds %d ints, need %d", a->stage_ints,
                  4 * a->n_new);

    // ---- plan (no caller state touched yet) ----
    // 64 blocks at a time: a word of wanted bits (from new_ids) against a word of resident bits (from
    // slot_of_block); only the set bits of the two differences are visited.
    const long long n_words = (a->n_blocks + 63) / 64;
    thread_local std::vector<unsigned long long> want;
    want.assign((size_t)n_words, 0ull);
    for (int k = 0; k < a->n_new; ++k) want[a->new_ids[k] >> 6] |= 1ull << (a->new_ids[k] & 63);
    std::vector<int>& leave = P->leave;
    std::vector<int>& enter = P->enter;
    leave.clear();
    enter.clear();
    int kept = 0, resident = 0;
    {
        // resident bits = sign bits of slot_of_block, four entries per SSE2 movemask; any entry below
        // -1 or at/above n_slots_total sets a lane of `bad`
        const int* sob = a->slot_of_block;
        const __m128i lo = _mm_set1_epi32(-1), hi = _mm_set1_epi32(a->n_slots_total - 1);
        __m128i bad = _mm_setzero_si128();
        for (long long wi = 0; wi < n_words; ++wi) {
            const long long b0 = 64 * wi;
            unsigned long long neg = 0ull;
            if (b0 + 64 <= a->n_blocks) {
                for (int i = 0; i < 16; ++i) {
                    const __m128i v = _mm_loadu_si128(reinterpret_cast<const __m128i*>(sob + b0 + 4 * i));
                    neg |= (unsigned long long)_mm_movemask_ps(_mm_castsi128_ps(v)) << (4 * i);
                    bad = _mm_or_si128(bad, _mm_or_si128(_mm_cmplt_epi32(v, lo), _mm_cmpgt_epi32(v, hi)));
                }
            } else {
                neg = ~0ull;
                for (long long b = b0; b < a->n_blocks; ++b) {
                    const int sv = sob[b];
                    if (sv >= 0) neg &= ~(1ull << (b - b0));
                    if (sv < -1 || sv >= a->n_slots_total) bad = _mm_set1_epi32(-1);
                }
            }
            const unsigned long long res = ~neg, w = want[wi];
            resident += __builtin_popcountll(res);
            kept += __builtin_popcountll(res & w);
            for (unsigned long long x = res & ~w; x; x &= x - 1) leave.push_back((int)(b0 + __builtin_ctzll(x)));
            for (unsigned long long x = w & ~res; x; x &= x - 1) enter.push_back((int)(b0 + __builtin_ctzll(x)));
        }
        if (_mm_movemask_epi8(bad)) {
            for (long long b = 0; b < a->n_blocks; ++b)
                LSA_CHECK_ARG(sob[b] >= -1 && sob[b] < a->n_slots_total,
                              "lsa_gather_blocks: slot_of_block[%lld]=%d (want -1 or a slot below %d)", b, sob[b],
                              a->n_slots_total);
        }
    }
    LSA_CHECK_ARG(resident + *a->n_free == a->capacity,
                  "lsa_gather_blocks: %d resident blocks + %d free slots != capacity %d", resident, *a->n_free,
                  a->capacity);
    const int avail = *a->n_free + (int)leave.size();
    if ((int)enter.size() > avail)
        return fail(LSA_ERR_CAPACITY, "lsa_gather_blocks: %zu entering blocks, %d slots available", enter.size(), avail);

    bool cold_host = false, stage_host = false;
    lsa_status st = device_view(a->cold, "lsa_gather_blocks", "cold", &P->cold_dev, &cold_host);
    if (st != LSA_OK) return st;
    st = device_view(a->stage, "lsa_gather_blocks", "stage", &P->stage_dev, &stage_host);
    if (st != LSA_OK) return st;
    LSA_CHECK_ARG(stage_host, "lsa_gather_blocks: stage must be pinned host memory");

    // Slot assignment without copying the free stack: conceptually the blocks that left push their
    // slots (ascending block id) on top of the caller's stack and each entering block (ascending)
    // pops the top, so entering block k takes entry n_free + n_leave - 1 - k of that stack.
    const int n_free = *a->n_free;
    const int n_leave = (int)leave.size();
    const int n_copies = (int)enter.size();
    std::vector<int>& leave_slot = P->freestack;  // slots of the blocks that left, in that order
    std::vector<int>& new_slot = P->new_slot;
    leave_slot.resize(n_leave);
    for (int j = 0; j < n_leave; ++j) leave_slot[j] = a->slot_of_block[leave[j]];
    new_slot.resize(n_copies);
    for (int k = 0; k < n_copies; ++k) {
        const int idx = n_free + n_leave - 1 - k;
        new_slot[k] = idx >= n_free ? leave_slot[idx - n_free] : a->free_slots[idx];
        LSA_CHECK_ARG(new_slot[k] >= 0 && new_slot[k] < a->n_slots_total, "lsa_gather_blocks: free slot %d out of range",
                      new_slot[k]);
    }
    // copy list then table, built in ordinary memory and moved to the pinned stage in one copy
    std::vector<int>& out = P->stage_buf;
    out.resize(2 * (size_t)(n_copies + a->n_new));
    for (int k = 0; k < n_copies; ++k) {
        out[2 * k] = enter[k];
        out[2 * k + 1] = new_slot[k];
    }
    {
        int* table = out.data() + 2 * n_copies;
        int e = 0;
        for (int k = 0; k < a->n_new; ++k) {
            const int b = a->new_ids[k];
            const int sl = a->slot_of_block[b];
            const int fresh = sl < 0;  // enter is the ascending list of new ids with no slot
            const int cand = n_copies > 0 ? new_slot[std::min(e, n_copies - 1)] : -1;  // in bounds either way
            table[2 * k] = b;
            table[2 * k + 1] = fresh ? cand : sl;
            e += fresh;
        }
    }
    std::memcpy(a->stage, out.data(), out.size() * sizeof(int));
    P->kept = kept;
    return LSA_OK;
}

// Apply a planned gather to the caller's state (after its copy kernel was enqueued).
void commit_gather(const lsa_gather_args* a, const GatherPlan& P) {
    for (int b : P.leave) a->slot_of_block[b] = -1;
    for (size_t k = 0; k < P.enter.size(); ++k) a->slot_of_block[P.enter[k]] = P.new_slot[k];
    // new stack = old entries 0 .. n_free-1, then the left slots, minus the n_enter popped from the top
    const int n_free = *a->n_free;
    const int top = n_free + (int)P.freestack.size() - (int)P.enter.size();
    for (int i = n_free; i < top; ++i) a->free_slots[i] = P.freestack[i - n_free];
    *a->n_free = top;
    *a->n_copied = (int)P.enter.size();
    *a->n_kept = P.kept;
}

// Plan every request, then launch the copy kernel(s), then commit: all or nothing.
lsa_status gather_batch(const lsa_gather_args* args, int n, hipStream_t stream) {
    LSA_CHECK_ARG(args != nullptr, "lsa_gather_blocks: null args");
    LSA_CHECK_ARG(n >= 1 && n <= LSA_MAX_REFRESH_REQ, "lsa_gather_blocks_batch: n=%d outside 1..%d", n,
                  LSA_MAX_REFRESH_REQ);
    for (int i = 0; i < n; ++i)
        for (int k = 0; k < i; ++k)
            LSA_CHECK_ARG(args[i].slot_of_block != args[k].slot_of_block && args[i].stage != args[k].stage,
                          "lsa_gather_blocks_batch: requests %d and %d share residency state or a staging buffer", k, i);
    thread_local std::vector<GatherPlan> plans;
    if ((int)plans.size() < n) plans.resize(n);
    for (int i = 0; i < n; ++i) {
        lsa_status st = plan_gather(&args[i], &plans[i]);
        if (st != LSA_OK) return st;
        LSA_CHECK_ARG(args[i].block_bytes == args[0].block_bytes, "lsa_gather_blocks_batch: block_bytes differ");
    }
    DeviceInfo dev;
    lsa_status st = current_device(&dev);
    if (st != LSA_OK) return st;
    LSA_CHECK_SUP(args[0].block_bytes / 4096 == 4 || args[0].block_bytes / 4096 == 8 || args[0].block_bytes / 4096 == 16,
                  "lsa_gather_blocks: block_bytes=%d", args[0].block_bytes);
    thread_local std::vector<std::pair<GatherParams, int>> launches;
    launches.clear();
    for (int i0 = 0; i0 < n; i0 += kMaxBatch) {
        const int nj = std::min(kMaxBatch, n - i0);
        GatherParams gp{};
        gp.n_jobs = nj;
        gp.block_bytes = args[0].block_bytes;
        for (int j = 0; j < nj; ++j) {
            const lsa_gather_args* a = &args[i0 + j];
            const GatherPlan& P = plans[i0 + j];
            const int n_copies = (int)P.enter.size();
            gp.job[j].cold = static_cast<const char*>(P.cold_dev);
            gp.job[j].hot = static_cast<char*>(a->hot);
            gp.job[j].copies = static_cast<const int*>(P.stage_dev);
            gp.job[j].tsrc = static_cast<const int*>(P.stage_dev) + 2 * n_copies;
            gp.job[j].tdst = a->table_dev;
            const int layers = std::max(1, a->n_layers);
            gp.job[j].n_copies = n_copies;
            gp.job[j].cold_layer_bytes = layers > 1 ? a->cold_layer_bytes : 0;
            gp.job[j].hot_layer_bytes = layers > 1 ? a->hot_layer_bytes : 0;
            gp.copy_off[j + 1] = gp.copy_off[j] + n_copies * layers;
            gp.table_off[j + 1] = gp.table_off[j] + a->n_new;
        }
        const int n_copies = gp.copy_off[nj], n_table = gp.table_off[nj];
        if (n_copies == 0 && n_table == 0) continue;
        // one group per copied block (capped), at least enough groups for the table copies
        const int grid = std::max(1, std::min(std::max(n_copies, (2 * n_table + 255) / 256), dev.cu_count * 32));
        launches.emplace_back(gp, grid);
    }
    // the caller's events (a[0]'s) take the dispatch stamps of the first and the last launch
    hipEvent_t ev0 = args[0].ev_begin, ev1 = args[0].ev_end;
    if (launches.empty()) {
        if (ev0) LSA_HIP(hipEventRecord(ev0, stream));
        if (ev1) LSA_HIP(hipEventRecord(ev1, stream));
    }
    for (size_t k = 0; k < launches.size(); ++k) {
        const GatherParams& gp = launches[k].first;
        const dim3 grid(launches[k].second), block(256);
        hipEvent_t b = k == 0 ? ev0 : nullptr, e = k + 1 == launches.size() ? ev1 : nullptr;
        // a launch that records events costs ~30 us of host time, a plain one ~3 us; after a
        // refresh the GPU waits for this launch, so events are taken only when asked for
        const int per = gp.block_bytes / 4096;
        if (b || e) {
            if (per == 4) hipExtLaunchKernelGGL(gather_kernel<4>, grid, block, 0, stream, b, e, 0, gp);
            else if (per == 8) hipExtLaunchKernelGGL(gather_kernel<8>, grid, block, 0, stream, b, e, 0, gp);
            else hipExtLaunchKernelGGL(gather_kernel<16>, grid, block, 0, stream, b, e, 0, gp);
        } else {
            if (per == 4) hipLaunchKernelGGL(gather_kernel<4>, grid, block, 0, stream, gp);
            else if (per == 8) hipLaunchKernelGGL(gather_kernel<8>, grid, block, 0, stream, gp);
            else hipLaunchKernelGGL(gather_kernel<16>, grid, block, 0, stream, gp);
        }
        LSA_HIP(hipGetLastError());
    }
    for (int i = 0; i < n; ++i) commit_gather(&args[i], plans[i]);
    return LSA_OK;
}

}  // namespace
}  // namespace lsa

using namespace lsa;

extern "C" lsa_status lsa_gather_blocks(const lsa_gather_args* a, hipStream_t stream) {
    return gather_batch(a, 1, stream);
}

extern "C" lsa_status lsa_gather_blocks_batch(const lsa_gather_args* a, int32_t n, hipStream_t stream) {
    return gather_batch(a, n, stream);
}
