// The gather planned on the device (zhichai.net explainer of "FlashMemory-DeepSeek-V4", section 2
// steps 3 and 5: the selected blocks are moved into GPU memory and the loaded set is refreshed),
// right after the refresh and with no host round trip.
//
// plan_kernel: one 1,024-thread group per request.  The refresh's union words are compared with the
// resident words: a counting pass checks that the new selection fits the request's slots (if not,
// nothing changes and the request's status is 1); then, in three ordered passes over the words (each
// a block-wide scan of per-word popcounts, so every block gets its rank in block-id order), the slots
// of blocks that left are pushed on the request's free stack, blocks that entered pop slots from the
// top (and are written to a copy list), and the table is rewritten in ascending block id while the
// resident words take the new selection.  A request whose refresh gave up (count -1) is left as it
// was (status 2).
// copy_kernel: every entering block (listed per request) copied cold -> hot for every layer, one
// 64-token block per group at a time; the number of blocks comes from the plan, on the device.
#include <hip/hip_ext.h>

#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int kMaxReq = LSA_MAX_REFRESH_REQ;
constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kCopyThreads = 256;

struct PlanParams {
    const unsigned long long* masks;
    int* sel_count;
    unsigned long long* resident;
    int* slot_of_block;
    int* free_slots;
    int* n_free;
    int2* table;
    int* table_count;
    int* copied;
    int* status;
    int* status_any;  // optional: OR of every status of the request since the caller cleared it
    int2* clist;  // copy list: request r's entering (block, slot) pairs from pair slot_off[r]
    int n_idx;
    long long blk_off[kMaxReq + 1];
    int word_off[kMaxReq + 1];
    int slot_off[kMaxReq + 1];
};

struct CopyParams {
    const char* cold[kMaxReq];
    char* hot;
    long long cold_layer_bytes, hot_layer_bytes;
    const int2* clist;
    const int* copied;
    const int* status;
    int slot_off[kMaxReq + 1];
    int n_req, n_layers, block_bytes;
};

// Exclusive scan of one int per thread over the group; *total receives the sum.
__device__ int group_exclusive_scan(int v, int* s_w, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
    }
    if (lane == 63) s_w[wave] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < kPlanWaves; ++k) {
        base += k < wave ? s_w[k] : 0;
        tot += s_w[k];
    }
    __syncthreads();  // s_w is reused by the next scan
    *total = tot;
    return base + inc - v;
}

__device__ int group_sum(int v, int* s_w) {
    int tot;
    group_exclusive_scan(v, s_w, &tot);
    return tot;
}

// The next (up to) kBits set bits of m, lowest first, cleared from m: their positions and how many.
// The passes below handle a word's blocks kBits at a time with every load of a batch issued before
// its stores (one memory round trip per batch instead of one per block); entries past the count
// repeat the first position, so those loads stay on a block of the word and their values go unused.
constexpr int kBits = 8;
__device__ __forceinline__ int take_bits(unsigned long long& m, int (&pos)[kBits]) {
    int n = 0;
#pragma unroll
    for (int k = 0; k < kBits; ++k) {
        pos[k] = m ? __ffsll((long long)m) - 1 : pos[0];
        n += m != 0ull;
        m &= m - 1ull;
    }
    return n;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanParams p) {
    __shared__ int s_w[kPlanWaves];
    const int r = blockIdx.x;
    const int W = p.word_off[r + 1] - p.word_off[r];
    const int s0 = p.slot_off[r];
    const unsigned long long* nm =
        p.masks + (size_t)(p.n_idx + 1) * p.word_off[r] + (size_t)p.n_idx * W;  // union plane
    unsigned long long* res = p.resident + p.word_off[r];
    int* sob = p.slot_of_block + p.blk_off[r];
    int* fs = p.free_slots + s0;
    int2* tbl = p.table + s0;
    int2* cl = p.clist + s0;

    int c_new = 0, c_enter = 0, c_leave = 0;
    // 2^lq threads per word when the request's words leave threads to spare (each takes a 64/2^lq
    // bit slice of its word, in order), so that a dense word's blocks take fewer dependent batches
    // in each pass; thread t handles word c0 + (t >> lq) of a chunk of wpc words
    const int lq = 4 * W <= kPlanThreads ? 2 : (2 * W <= kPlanThreads ? 1 : 0);
    const int wpc = kPlanThreads >> lq;
    const int tw = (int)threadIdx.x >> lq;
    const int sl = 64 >> lq;  // bits per slice
    const unsigned long long slice =
        lq == 0 ? ~0ull : (((1ull << sl) - 1ull) << (sl * ((int)threadIdx.x & ((1 << lq) - 1))));
    // a request of at most wpc words: each thread's word is the same in every pass, so it stays in
    // registers (one round trip fewer per pass); longer requests re-read their words
    const bool one = W <= wpc;
    unsigned long long u1 = 0ull, o1 = 0ull;
    if (one && tw < W) {
        u1 = nm[tw];
        o1 = res[tw];
    }
    auto new_word = [&](int w) { return one ? u1 : (w < W ? nm[w] : 0ull); };
    auto old_word = [&](int w) { return one ? o1 : (w < W ? res[w] : 0ull); };
    for (int c0 = 0; c0 < W; c0 += wpc) {
        const int w = c0 + tw;
        const unsigned long long u = new_word(w) & slice, o = old_word(w) & slice;
        c_new += __popcll(u);
        c_enter += __popcll(u & ~o);
        c_leave += __popcll(o & ~u);
    }
    const int n_new = group_sum(c_new, s_w);
    const int n_enter = group_sum(c_enter, s_w);
    const int n_leave = group_sum(c_leave, s_w);
    const int nf = p.n_free[r];
    const bool gave_up = p.sel_count[r] < 0;
    __syncthreads();  // every thread has read the count before it is rewritten below
    if (gave_up || n_enter > nf + n_leave) {  // nothing changes for this request
        if (threadIdx.x == 0) {
            p.sel_count[r] = gave_up ? 0 : n_new;
            p.status[r] = gave_up ? 2 : 1;
            if (p.status_any) p.status_any[r] |= gave_up ? 2 : 1;
            p.copied[r] = 0;
        }
        return;
    }
    // leaving blocks push their slots, in ascending block id
    int base = 0;
    for (int c0 = 0; c0 < W; c0 += wpc) {
        const int w = c0 + tw;
        unsigned long long m = old_word(w) & ~new_word(w) & slice;
        int tot;
        int at = base + group_exclusive_scan(__popcll(m), s_w, &tot);
        while (m) {
            int pos[kBits];
            const int n = take_bits(m, pos);
            int slot[kBits];
#pragma unroll
            for (int k = 0; k < kBits; ++k) slot[k] = sob[64 * w + pos[k]];
#pragma unroll
            for (int k = 0; k < kBits; ++k) {
                if (k < n) {
                    fs[nf + at + k] = slot[k];
                    sob[64 * w + pos[k]] = -1;
                }
            }
            at += n;
        }
        base += tot;
    }
    __syncthreads();
    // entering blocks pop slots from the top of the stack, in ascending block id
    const int nf2 = nf + n_leave;
    base = 0;
    for (int c0 = 0; c0 < W; c0 += wpc) {
        const int w = c0 + tw;
        unsigned long long m = new_word(w) & ~old_word(w) & slice;
        int tot;
        int e = base + group_exclusive_scan(__popcll(m), s_w, &tot);
        while (m) {
            int pos[kBits];
            const int n = take_bits(m, pos);
            int slot[kBits];
#pragma unroll
            for (int k = 0; k < kBits; ++k) slot[k] = fs[nf2 - 1 - (e + min(k, n - 1))];
#pragma unroll
            for (int k = 0; k < kBits; ++k) {
                if (k < n) {
                    const int id = 64 * w + pos[k];
                    sob[id] = slot[k];
                    cl[e + k] = make_int2(id, slot[k]);
                }
            }
            e += n;
        }
        base += tot;
    }
    __syncthreads();
    // the table in ascending block id; the resident words take the new selection
    base = 0;
    for (int c0 = 0; c0 < W; c0 += wpc) {
        const int w = c0 + tw;
        const unsigned long long u = new_word(w);
        unsigned long long m = u & slice;
        int tot;
        int at = base + group_exclusive_scan(__popcll(m), s_w, &tot);
        while (m) {
            int pos[kBits];
            const int n = take_bits(m, pos);
            int slot[kBits];
#pragma unroll
            for (int k = 0; k < kBits; ++k) slot[k] = sob[64 * w + pos[k]];
#pragma unroll
            for (int k = 0; k < kBits; ++k)
                if (k < n) tbl[at + k] = make_int2(64 * w + pos[k], slot[k]);
            at += n;
        }
        if (w < W && ((int)threadIdx.x & ((1 << lq) - 1)) == 0) res[w] = u;  // the word's first slice
        base += tot;
    }
    if (threadIdx.x == 0) {
        p.sel_count[r] = n_new;
        p.n_free[r] = nf2 - n_enter;
        p.table_count[r] = n_new;
        p.copied[r] = n_enter;
        p.status[r] = 0;
    }
}

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

// Copy c of the launch (the requests' entering blocks concatenated, layer-major) goes to group c,
// c + G, ...: 256 threads x 16-byte vectors, every load of a block in flight before its stores.
template <int PER>  // 16-byte vectors per thread per block (block_bytes / 4096)
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(CopyParams p) {
    __shared__ int s_pre[kMaxReq + 1];
    if (threadIdx.x == 0) {
        int run = 0;
        for (int r = 0; r < p.n_req; ++r) {
            s_pre[r] = run;
            run += p.status[r] == 0 ? p.copied[r] : 0;
        }
        s_pre[p.n_req] = run;
    }
    __syncthreads();
    const int per_layer = s_pre[p.n_req];
    constexpr int STEP = PER > 8 ? 8 : PER;
    for (int c = blockIdx.x; c < per_layer * p.n_layers; c += gridDim.x) {
        const int layer = c / per_layer;
        const int k = c - layer * per_layer;
        int r = 0;
        while (r + 1 < p.n_req && s_pre[r + 1] <= k) ++r;
        const int2 pr = p.clist[p.slot_off[r] + (k - s_pre[r])];
        const uint4* src = reinterpret_cast<const uint4*>(p.cold[r] + layer * p.cold_layer_bytes +
                                                          (size_t)pr.x * p.block_bytes);
        uint4* dst = reinterpret_cast<uint4*>(p.hot + layer * p.hot_layer_bytes + (size_t)pr.y * p.block_bytes);
#pragma unroll
        for (int v0 = 0; v0 < PER; v0 += STEP) {
            uint4 b[STEP];
#pragma unroll
            for (int v = 0; v < STEP; ++v) b[v] = load_nt(src + (v0 + v) * kCopyThreads + threadIdx.x);
#pragma unroll
            for (int v = 0; v < STEP; ++v) store_nt(dst + (v0 + v) * kCopyThreads + threadIdx.x, b[v]);
        }
    }
}

__global__ void reset_kernel(unsigned long long* resident, long long n_words, int* slot_of_block, long long n_blocks,
                             int* free_slots, int n_slots, const int* slot_off_dev, int n_req, int* n_free,
                             int* table_count, int* status) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n_words) resident[i] = 0ull;
    if (i < n_blocks) slot_of_block[i] = -1;
    if (i < n_slots) {
        // request of slot i: the last r with slot_off[r] <= i; its stack holds its slots top-down
        int r = 0;
        while (r + 1 < n_req && slot_off_dev[r + 1] <= i) ++r;
        const int lo = slot_off_dev[r], hi = slot_off_dev[r + 1];
        free_slots[i] = hi - 1 - (int)(i - lo);
    }
    if (i < n_req) {
        n_free[i] = slot_off_dev[i + 1] - slot_off_dev[i];
        table_count[i] = 0;
        status[i] = 0;
    }
}

struct ResidencyPlan {
    long long n_blocks = 0, n_words = 0;
    int n_slots = 0;
    size_t total = 0;  // workspace: copy list, then a copy of slot_off for the reset
};

lsa_status residency_check(const lsa_device_gather_args* a, ResidencyPlan* P) {
    LSA_CHECK_ARG(a != nullptr, "lsa_gather_plan_device: null args");
    LSA_CHECK_ARG(a->n_req >= 1 && a->n_req <= kMaxReq, "lsa_gather_plan_device: n_req=%d outside 1..%d", a->n_req,
                  kMaxReq);
    LSA_CHECK_SUP(a->n_idx >= 1 && a->n_idx <= 4, "lsa_gather_plan_device: n_idx=%d (1..4)", a->n_idx);
    LSA_CHECK_SUP(a->block_bytes == 16384 || a->block_bytes == 32768 || a->block_bytes == 65536,
                  "lsa_gather_plan_device: block_bytes=%d", a->block_bytes);
    LSA_CHECK_ARG(a->n_layers >= 1 && a->n_layers <= 256, "lsa_gather_plan_device: n_layers=%d outside 1..256",
                  a->n_layers);
    LSA_CHECK_ARG(a->blk_off && a->slot_off, "lsa_gather_plan_device: blk_off / slot_off is null");
    LSA_CHECK_ARG(a->blk_off[0] == 0 && a->slot_off[0] == 0, "lsa_gather_plan_device: offsets must start at 0");
    long long words = 0;
    for (int r = 0; r < a->n_req; ++r) {
        const long long nb = a->blk_off[r + 1] - a->blk_off[r];
        const long long ns = (long long)a->slot_off[r + 1] - a->slot_off[r];
        LSA_CHECK_ARG(nb >= 1 && nb <= (1ll << 24), "lsa_gather_plan_device: request %d has %lld blocks", r, nb);
        LSA_CHECK_ARG(ns >= 0, "lsa_gather_plan_device: request %d has %lld slots", r, ns);
        words += (nb + 63) / 64;
    }
    LSA_CHECK_ARG(words <= (1ll << 26) && a->slot_off[a->n_req] <= (1 << 30),
                  "lsa_gather_plan_device: too many blocks or slots");
    if (a->n_layers > 1) {
        LSA_CHECK_ARG(a->cold_layer_bytes % 16 == 0 && a->hot_layer_bytes % 16 == 0 &&
                          a->hot_layer_bytes >= (long long)a->slot_off[a->n_req] * a->block_bytes,
                      "lsa_gather_plan_device: layer strides");
    }
    P->n_blocks = a->blk_off[a->n_req];
    P->n_words = words;
    P->n_slots = a->slot_off[a->n_req];
    P->total = align_up((size_t)std::max(1, P->n_slots) * sizeof(int2), 256) + align_up((kMaxReq + 1) * sizeof(int), 256);
    return LSA_OK;
}

lsa_status residency_state_check(const lsa_device_gather_args* a) {
    LSA_CHECK_ARG(a->resident && a->slot_of_block && a->free_slots && a->n_free && a->table_count && a->status,
                  "lsa_gather_plan_device: null state pointer");
    return LSA_OK;
}

}  // namespace
}  // namespace lsa

using namespace lsa;

extern "C" lsa_status lsa_gather_plan_device_workspace(const lsa_device_gather_args* a, size_t* bytes) {
    ResidencyPlan P;
    lsa_status st = residency_check(a, &P);
    if (st != LSA_OK) return st;
    LSA_CHECK_ARG(bytes != nullptr, "lsa_gather_plan_device_workspace: bytes is null");
    *bytes = P.total;
    return LSA_OK;
}

extern "C" lsa_status lsa_gather_plan_device(const lsa_device_gather_args* a, hipStream_t stream) {
    ResidencyPlan P;
    lsa_status st = residency_check(a, &P);
    if (st != LSA_OK) return st;
    st = residency_state_check(a);
    if (st != LSA_OK) return st;
    LSA_CHECK_ARG(a->masks && a->sel_count && a->hot && a->table && a->copied && a->cold,
                  "lsa_gather_plan_device: null pointer");
    for (int r = 0; r < a->n_req; ++r) LSA_CHECK_ARG(a->cold[r] != nullptr, "lsa_gather_plan_device: cold[%d] is null", r);
    if (a->workspace == nullptr || a->workspace_bytes < P.total)
        return fail(LSA_ERR_WORKSPACE, "lsa_gather_plan_device: workspace of %zu bytes, need %zu",
                    a->workspace ? a->workspace_bytes : (size_t)0, P.total);
    LSA_CHECK_ARG(((uintptr_t)a->hot % 16) == 0 && ((uintptr_t)a->table % 8) == 0 && ((uintptr_t)a->workspace % 16) == 0,
                  "lsa_gather_plan_device: hot (16 B), table (8 B) and workspace (16 B) alignment");
    // the last check, the first HIP call: each cold pool in HBM or in pinned host memory (then the copy kernel reads it over the host link)
    const char* cold_dev[LSA_MAX_REFRESH_REQ];
    for (int r = 0; r < a->n_req; ++r) {
        const void* d = nullptr;
        bool host = false;
        st = device_view(a->cold[r], "lsa_gather_plan_device", "cold[r]", &d, &host);
        if (st != LSA_OK) return st;
        cold_dev[r] = static_cast<const char*>(d);
    }
    PlanParams pp;
    pp.masks = reinterpret_cast<const unsigned long long*>(a->masks);
    pp.sel_count = a->sel_count;
    pp.resident = reinterpret_cast<unsigned long long*>(a->resident);
    pp.slot_of_block = a->slot_of_block;
    pp.free_slots = a->free_slots;
    pp.n_free = a->n_free;
    pp.table = reinterpret_cast<int2*>(a->table);
    pp.table_count = a->table_count;
    pp.copied = a->copied;
    pp.status = a->status;
    pp.status_any = a->status_any;
    pp.clist = static_cast<int2*>(a->workspace);
    pp.n_idx = a->n_idx;
    int wo = 0;
    for (int r = 0; r <= a->n_req; ++r) {
        pp.blk_off[r] = a->blk_off[r];
        pp.word_off[r] = wo;
        pp.slot_off[r] = a->slot_off[r];
        if (r < a->n_req) wo += (int)((a->blk_off[r + 1] - a->blk_off[r] + 63) / 64);
    }
    // events only when asked for: a launch that records them costs ~30 us of host time
    if (a->ev_begin)
        hipExtLaunchKernelGGL(plan_kernel, dim3(a->n_req), dim3(kPlanThreads), 0, stream, a->ev_begin, nullptr, 0, pp);
    else
        hipLaunchKernelGGL(plan_kernel, dim3(a->n_req), dim3(kPlanThreads), 0, stream, pp);
    LSA_HIP(hipGetLastError());
    CopyParams cp;
    for (int r = 0; r < a->n_req; ++r) cp.cold[r] = cold_dev[r];
    cp.hot = static_cast<char*>(a->hot);
    cp.cold_layer_bytes = a->n_layers > 1 ? a->cold_layer_bytes : 0;
    cp.hot_layer_bytes = a->n_layers > 1 ? a->hot_layer_bytes : 0;
    cp.clist = pp.clist;
    cp.copied = a->copied;
    cp.status = a->status;
    for (int r = 0; r <= a->n_req; ++r) cp.slot_off[r] = a->slot_off[r];
    cp.n_req = a->n_req;
    cp.n_layers = a->n_layers;
    cp.block_bytes = a->block_bytes;
    DeviceInfo dev;
    st = current_device(&dev);
    if (st != LSA_OK) return st;
    const dim3 grid(dev.cu_count * 8), block(kCopyThreads);
    switch (a->block_bytes / (kCopyThreads * 16)) {
        case 4:
            if (a->ev_end) hipExtLaunchKernelGGL(copy_kernel<4>, grid, block, 0, stream, nullptr, a->ev_end, 0, cp);
            else hipLaunchKernelGGL(copy_kernel<4>, grid, block, 0, stream, cp);
            break;
        case 8:
            if (a->ev_end) hipExtLaunchKernelGGL(copy_kernel<8>, grid, block, 0, stream, nullptr, a->ev_end, 0, cp);
            else hipLaunchKernelGGL(copy_kernel<8>, grid, block, 0, stream, cp);
            break;
        default:
            if (a->ev_end) hipExtLaunchKernelGGL(copy_kernel<16>, grid, block, 0, stream, nullptr, a->ev_end, 0, cp);
            else hipLaunchKernelGGL(copy_kernel<16>, grid, block, 0, stream, cp);
            break;
    }
    LSA_HIP(hipGetLastError());
    return LSA_OK;
}

extern "C" lsa_status lsa_residency_reset(const lsa_device_gather_args* a, hipStream_t stream) {
    ResidencyPlan P;
    lsa_status st = residency_check(a, &P);
    if (st != LSA_OK) return st;
    st = residency_state_check(a);
    if (st != LSA_OK) return st;
    if (a->workspace == nullptr || a->workspace_bytes < P.total)
        return fail(LSA_ERR_WORKSPACE, "lsa_residency_reset: workspace of %zu bytes, need %zu",
                    a->workspace ? a->workspace_bytes : (size_t)0, P.total);
    // slot offsets for the kernel: through the workspace tail, from a host copy kept alive until the
    // copy has run (a synchronous copy: the reset happens once, at set-up)
    int* off_dev = reinterpret_cast<int*>(static_cast<char*>(a->workspace) +
                                          align_up((size_t)std::max(1, P.n_slots) * sizeof(int2), 256));
    LSA_HIP(hipMemcpyAsync(off_dev, a->slot_off, (a->n_req + 1) * sizeof(int), hipMemcpyHostToDevice, stream));
    LSA_HIP(hipStreamSynchronize(stream));
    const long long n = std::max<long long>({P.n_words, P.n_blocks, (long long)P.n_slots, (long long)a->n_req});
    hipLaunchKernelGGL(reset_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<unsigned long long*>(a->resident), P.n_words, a->slot_of_block, P.n_blocks,
                       a->free_slots, P.n_slots, off_dev, a->n_req, a->n_free, a->table_count, a->status);
    LSA_HIP(hipGetLastError());
    return LSA_OK;
}
