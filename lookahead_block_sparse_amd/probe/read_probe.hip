// Read-bandwidth probe: how fast one launch can stream a region of device memory that is in no
// cache, with the access patterns and launch shapes of the index refresh and the attention kernel.
// It computes nothing (each wave folds its loads into one word that is stored only if it equals a
// value the caller picks), and is built as its own library, apart from the LSA path.
//
// A batch is `loads` KiB: `loads` load instructions per lane of 16 bytes each.
//   pattern 0 ("runs"): load j of a batch reads the j-th 1 KiB run whole (lane l: bytes 16 l ..).
//   pattern 1 ("rows"): a batch is loads/16 units of 32 rows x 512 bytes; load j = 4 g + k of a
//                      unit reads 128 bytes (slice k) of each of rows 8 g .. 8 g + 7 (lane l: row
//                      8 g + l / 8, bytes 128 k + 16 (l % 8)), the index refresh's key pattern.
// Wave w of W takes batches w, w + W, ...; every load of a batch is issued before any is used.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
}

template <int L, int PATTERN, bool NT>
__global__ __launch_bounds__(256) void read_kernel(const char* __restrict__ buf, long long n_batches,
                                                   unsigned* __restrict__ sink, unsigned magic) {
    const int lane = threadIdx.x & 63;
    const long long waves = (long long)gridDim.x * (blockDim.x >> 6);
    const long long w0 = (long long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (long long b = w0; b < n_batches; b += waves) {
        const char* base = buf + b * (long long)L * 1024;
        u32x4 v[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            long long off;
            if constexpr (PATTERN == 0) {
                off = (long long)j * 1024 + lane * 16;
            } else {
                const int unit = j / 16, g = (j % 16) / 4, k = j % 4;
                off = (long long)unit * 16384 + (g * 8 + (lane >> 3)) * 512 + k * 128 + (lane & 7) * 16;
            }
            v[j] = ld<NT>(reinterpret_cast<const u32x4*>(base + off));
        }
        __builtin_amdgcn_sched_barrier(0);  // every load of the batch is issued before the first use
#pragma unroll
        for (int j = 0; j < L; ++j) acc ^= v[j];
    }
    if (acc.x == magic && acc.y == magic && acc.z == magic && acc.w == magic)
        sink[w0 * 64 + lane] = acc.x;
}

template <int L, int PATTERN, bool NT>
hipError_t launch(const void* buf, long long n_batches, int groups, unsigned* sink, unsigned magic,
                  hipEvent_t e0, hipEvent_t e1, hipStream_t s) {
    const dim3 grid(groups), block(256);
    const char* b = static_cast<const char*>(buf);
    if (e0 && e1)
        hipExtLaunchKernelGGL((read_kernel<L, PATTERN, NT>), grid, block, 0, s, e0, e1, 0, b, n_batches, sink, magic);
    else
        hipLaunchKernelGGL((read_kernel<L, PATTERN, NT>), grid, block, 0, s, b, n_batches, sink, magic);
    return hipGetLastError();
}

typedef hipError_t (*launch_fn)(const void*, long long, int, unsigned*, unsigned, hipEvent_t, hipEvent_t,
                                hipStream_t);

template <int PATTERN, bool NT>
launch_fn pick_l(int loads) {
    switch (loads) {
        case 16: return launch<16, PATTERN, NT>;
        case 32: return launch<32, PATTERN, NT>;
        case 48: return launch<48, PATTERN, NT>;
        default: return nullptr;
    }
}

launch_fn pick(int pattern, int loads, int nt) {
    if (pattern == 0) return nt ? pick_l<0, true>(loads) : pick_l<0, false>(loads);
    if (pattern == 1) return nt ? pick_l<1, true>(loads) : pick_l<1, false>(loads);
    return nullptr;
}

}  // namespace

extern "C" {

// Batches of one launch over `bytes` (the tail that does not fill a batch is not read).
long long probe_batches(long long bytes, int loads) { return loads > 0 ? bytes / ((long long)loads * 1024) : 0; }

// Work-groups of 4 waves that fit one compute unit at once for this variant (0 if unknown variant).
int probe_groups_per_cu(int pattern, int loads, int nontemporal) {
    launch_fn f = pick(pattern, loads, nontemporal);
    if (!f) return 0;
    int n = 0;
    hipError_t e = hipSuccess;
#define PROBE_OCC(P, LL, N)                                                                           \
    if (pattern == P && loads == LL && (nontemporal != 0) == N)                                      \
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, read_kernel<LL, P, N>, 256, 0);
    PROBE_OCC(0, 16, false) PROBE_OCC(0, 32, false) PROBE_OCC(0, 48, false)
    PROBE_OCC(0, 16, true) PROBE_OCC(0, 32, true) PROBE_OCC(0, 48, true)
    PROBE_OCC(1, 16, false) PROBE_OCC(1, 32, false) PROBE_OCC(1, 48, false)
    PROBE_OCC(1, 16, true) PROBE_OCC(1, 32, true) PROBE_OCC(1, 48, true)
#undef PROBE_OCC
    return e == hipSuccess ? n : 0;
}

// One read of buf[0 .. probe_batches(bytes, loads) * loads KiB) on `stream`.  groups = 0 launches
// one wave per batch (every load of the launch issued at once); otherwise `groups` 4-wave groups
// loop over the batches.  sink: device, >= 64 * 4 * (launched groups) words.  The events, when
// both are given, take the dispatch's start and end stamps.  Returns 0, -1 for bad arguments, or
// the HIP error code of the launch.
int probe_read(const void* buf, long long bytes, int pattern, int loads, int nontemporal, int groups,
               unsigned* sink, unsigned magic, hipEvent_t ev0, hipEvent_t ev1, hipStream_t stream) {
    launch_fn f = pick(pattern, loads, nontemporal);
    const long long nb = probe_batches(bytes, loads);
    if (!f || !buf || !sink || nb <= 0 || groups < 0 || ((uintptr_t)buf % 1024) != 0) return -1;
    if (pattern == 1 && loads % 16 != 0) return -1;
    const long long g = groups > 0 ? groups : (nb + 3) / 4;
    if (g > (1ll << 30)) return -1;
    const hipError_t e = f(buf, nb, (int)g, sink, magic, ev0, ev1, stream);
    return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
