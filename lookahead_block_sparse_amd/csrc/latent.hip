// Low-rank query projection, first factor: the latent c_i = A_i h of every indexer (zhichai.net
// explainer of "FlashMemory-DeepSeek-V4", section 4, training tricks: a query projection of rank
// 2048 through the backbone's MLA/MQA bottleneck).  The refresh's Query Encoder then projects the
// latent with B_i.
//
// A GEMV over A [n_idx][rank][d_model] shared by every request, HBM-bound on A (25 M elements at
// n_idx = 3, r = 2048, d = 4096), read once per call for all requests.  A work-group owns a tile of
// kG consecutive rows of A (all of one indexer); its waves split the row into slices of 64 16-byte
// chunks: lane l of the wave on slice s holds chunk 64 s + l of each of the kG rows, so that one load
// instruction reads a contiguous 1 KiB run, and all kG loads of a wave are issued before any use.
// The A chunks stay in registers while the requests go by kQ at a time: the lane loads its chunk of
// each request's hidden state (L2-resident, 16 bytes per request), forms the kG x kQ partial dot
// products (fp32 accumulation), and a butterfly reduce-scatter across the wave leaves each lane one
// of those sums; the slices' sums meet in LDS, and the latent is stored in the input type (bf16:
// round to nearest, ties to even).
#include <hip/hip_ext.h>

#include <algorithm>
#include <type_traits>

#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int kMaxReq = LSA_MAX_REFRESH_REQ;
constexpr int kMaxWaves = 8;  // slices handled side by side; wider rows loop over slices
constexpr int kG = 16;        // rows of A per tile (rank is a multiple of 256: tiles never straddle indexers)
constexpr int kQ = 2;         // requests per round
constexpr int kN = kG * kQ;   // partial sums per lane per round (a power of two, at most 64)
static_assert((kN & (kN - 1)) == 0 && kN <= 64, "reduce-scatter over a power of two");

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// A is read once per call, through a buffer resource over the tile: non-temporal 16-byte loads at
// a per-row scalar offset plus the lane's offset, so that all loads of a tile share one address
// register (and a load past the tile returns zeros instead of touching memory).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 load_nt(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2 /* nt */);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint4 load(const char* base, unsigned off) {
    return *reinterpret_cast<const uint4*>(base + off);
}

struct LatentParams {
    const void* hidden;
    long long hidden_req_stride, hidden_idx_stride;
    const void* w_down;
    void* latent;
    int n_req, d_model, rank, n_idx;
};

template <typename T>
struct Elem;
template <>
struct Elem<uint16_t> {
    static constexpr int N = 8;  // elements per 16 bytes
    // a.b over 8 bf16 pairs with the packed dot of two bf16 pairs into fp32 (v_dot2_f32_bf16: the
    // products of bf16 values are exact in fp32), 4 instructions where unpacking and fusing take 24
    __device__ static float dot(uint4 a, uint4 b) {
        float acc = __builtin_amdgcn_fdot2_f32_bf16(bf2(a.x), bf2(b.x), 0.0f, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(bf2(a.y), bf2(b.y), acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(bf2(a.z), bf2(b.z), acc, false);
        return __builtin_amdgcn_fdot2_f32_bf16(bf2(a.w), bf2(b.w), acc, false);
    }
    __device__ static bf16x2 bf2(unsigned w) { return __builtin_bit_cast(bf16x2, w); }
    // round to nearest, ties to even: add 0x7fff plus the lowest kept bit, keep the high half
    __device__ static uint16_t store(float x) {
        const unsigned b = __float_as_uint(x);
        return (uint16_t)((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
    }
};
template <>
struct Elem<float> {
    static constexpr int N = 4;
    __device__ static float dot(uint4 a, uint4 b) {
        float acc = __uint_as_float(a.x) * __uint_as_float(b.x);
        acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
        acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
        return fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
    }
    __device__ static float store(float x) { return x; }
};

// v[0 .. kN) summed over the 64 lanes, scattered: afterwards v[0] of lane l holds the sum of entry
// l mod kN.  At offset o every lane pairs with a lane whose index differs in bit o and agrees in
// the bits above it; the lane keeps the half of its 2o entries that bit o of its own index selects
// and adds the partner's copy of that half.  The exchanges are full-rate cross-lane moves: the
// 16-lane row swap at o = 16, the row mirror (lane ^ 15) at 8, the half-row mirror (lane ^ 7) at 4,
// quad permutations at 2 and 1, and the half-wave swap for the final sum.
__device__ __forceinline__ float as_f(unsigned x) { return __uint_as_float(x); }
__device__ __forceinline__ unsigned as_u(float x) { return __float_as_uint(x); }
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <int O, int CTRL>
__device__ __forceinline__ void pair_step(float (&v)[kN], int lane) {
    const bool hi = (lane & O) != 0;
#pragma unroll
    for (int j = 0; j < O; ++j) {
        const float keep = hi ? v[j + O] : v[j];
        const float send = hi ? v[j] : v[j + O];
        v[j] = keep + dpp<CTRL>(send);
    }
}
__device__ __forceinline__ void reduce_scatter(float (&v)[kN], int lane) {
    static_assert(kN == 32, "the exchange pattern below covers 32 entries");
#pragma unroll
    for (int j = 0; j < 16; ++j) {  // odd rows of v[j] trade with even rows of v[j + 16]
        const auto r = __builtin_amdgcn_permlane16_swap(as_u(v[j]), as_u(v[j + 16]), false, false);
        v[j] = as_f(r[0]) + as_f(r[1]);
    }
    pair_step<8, 0x140>(v, lane);  // row_mirror
    pair_step<4, 0x141>(v, lane);  // row_half_mirror
    pair_step<2, 0x4E>(v, lane);   // quad_perm [2, 3, 0, 1]
    pair_step<1, 0xB1>(v, lane);   // quad_perm [1, 0, 3, 2]
    const auto r = __builtin_amdgcn_permlane32_swap(as_u(v[0]), as_u(v[0]), false, false);
    v[0] = as_f(r[0]) + as_f(r[1]);
}

// grid: one work-group per tile of kG rows; block: 64 x min(slices, kMaxWaves) threads; LDS:
// rounds x waves x kN floats
template <typename T>
__global__ __launch_bounds__(64 * kMaxWaves) void latent_kernel(LatentParams p) {
    using E = Elem<T>;
    extern __shared__ float part[];  // [round][wave][kN]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_waves = blockDim.x >> 6;
    const int hc = p.d_model / E::N;  // 16-byte chunks per row
    const int n_slices = (hc + 63) / 64;
    const int rounds = (p.n_req + kQ - 1) / kQ;
    const int row0 = blockIdx.x * kG;  // over n_idx * rank rows
    const int i = row0 / p.rank;
    const size_t row_bytes = (size_t)p.d_model * sizeof(T);
    const __amdgpu_buffer_rsrc_t a = tile_rsrc(static_cast<const char*>(p.w_down) + (size_t)row0 * row_bytes,
                                               (unsigned)(kG * row_bytes));
    const char* hid = static_cast<const char*>(p.hidden) + (size_t)i * p.hidden_idx_stride * sizeof(T);
    const size_t req_bytes = (size_t)p.hidden_req_stride * sizeof(T);
    for (int s = wave; s < n_slices; s += n_waves) {
        const int c = s * 64 + lane;
        const bool live = c < hc;  // a bf16 row of 256 (2k+1) elements ends in half a slice
        const unsigned off = (unsigned)(live ? c : hc - 1) * 16u;
        uint4 av[kG];
#pragma unroll
        for (int g = 0; g < kG; ++g) av[g] = load_nt(a, off, (unsigned)(g * row_bytes));
        if (!live)  // dead lanes add exact zeros
#pragma unroll
            for (int g = 0; g < kG; ++g) av[g] = make_uint4(0, 0, 0, 0);
        // the next round's hidden chunks are requested before this round's sums (L2 latency hidden)
        uint4 hv[kQ], hn[kQ];
#pragma unroll
        for (int q = 0; q < kQ; ++q) hv[q] = load(hid + min(q, p.n_req - 1) * req_bytes, off);
        for (int rd = 0; rd < rounds; ++rd) {
#pragma unroll
            for (int q = 0; q < kQ; ++q) hn[q] = load(hid + min((rd + 1) * kQ + q, p.n_req - 1) * req_bytes, off);
            if (!live)
#pragma unroll
                for (int q = 0; q < kQ; ++q) hv[q] = make_uint4(0, 0, 0, 0);
            float v[kN];
#pragma unroll
            for (int g = 0; g < kG; ++g)
#pragma unroll
                for (int q = 0; q < kQ; ++q) v[g * kQ + q] = E::dot(av[g], hv[q]);
            reduce_scatter(v, lane);
            if (lane < kN) {
                float* d = part + ((size_t)rd * n_waves + wave) * kN + lane;
                *d = s == wave ? v[0] : *d + v[0];  // later slices of this wave add to their own entry
            }
#pragma unroll
            for (int q = 0; q < kQ; ++q) hv[q] = hn[q];
        }
    }
    __syncthreads();
    T* out = static_cast<T*>(p.latent);
    const int k0 = row0 - i * p.rank;
    for (int o = threadIdx.x; o < rounds * kN; o += blockDim.x) {
        const int rd = o / kN, e = o % kN;
        const int w_used = min(n_waves, n_slices);
        float sum = 0.0f;
        for (int w = 0; w < w_used; ++w) sum += part[((size_t)rd * n_waves + w) * kN + e];
        const int g = e / kQ, r = rd * kQ + e % kQ;
        if (r < p.n_req) out[((size_t)r * p.n_idx + i) * p.rank + k0 + g] = E::store(sum);
    }
}

// Matrix-core variant for batches of requests (bf16): per work-group a tile of 16 rows of A
// against 16 requests at a time, v_mfma_f32_16x16x32_bf16 with A's rows and the requests' hidden
// states as the two operands.  Lane l supplies row l % 16 of A and request l % 16 of the block, both
// at the same 8 elements of each 32-element step (chunk l / 16 of the step's four), so every product
// pairs an element of A with the hidden state's element of the same dimension, whatever the order
// inside the instruction.  As in the vector kernel the waves split the row into slices of 64
// chunks, whose 16 loads of A per lane stay in registers while the request blocks go by; the slices
// meet in LDS.  A's operand arrives straight from memory (16 rows x 64 bytes a load, each row
// streamed once); the hidden states, which every work-group reads, go through a per-wave LDS tile
// instead: a quarter slice (16 chunks) of the block's 16 requests is loaded as 4 runs of 256
// contiguous bytes per instruction, written to the tile and read back in operand order.  Loaded in
// operand order (16 pieces of 64 bytes a load, a request stride apart) they made up most of the
// kernel's time at 64 requests; through the tile the LDS round trip is what remains of their cost.
// The tile's chunks are XOR-swizzled by request, so both the writes and the reads touch 16
// distinct 16-byte bank groups per 16 lanes.  The next quarter's loads are in flight while the
// current one is read and multiplied (a second quarter in flight measured no faster).
// The vector kernel turns ALU-bound beyond a few requests (its dot products and reduce-scatters grow
// with the batch), the matrix cores do not.
constexpr int kMfmaMinReq = 10;  // batches from this size take the matrix cores
constexpr int kMSteps = 16;     // 32-element steps per slice (64 chunks of 16 bytes)
// Chunks past a short row's end load from this offset, beyond both buffer ranges (< 2^30 bytes), so
// they read as zeros without a wait; adding up to 64 request strides (< 2^24 bytes) stays below 2^32.
constexpr unsigned kPastEnd = 0xC0000000u;
constexpr size_t kMfmaMaxReqBytes = (size_t)1 << 24;  // hidden-state stride bound for the matrix cores
constexpr size_t kMfmaMaxRange = (size_t)1 << 30;     // hidden-state range bound for the matrix cores

__global__ __launch_bounds__(64 * kMaxWaves) void latent_mfma_kernel(LatentParams p) {
    // [request block][wave][16 rows][16 requests] partial sums, then one 16 x 16-chunk B tile per wave
    extern __shared__ float mpart[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_waves = blockDim.x >> 6;
    const int rl = lane & 15, kc = lane >> 4;
    const int hc = p.d_model / 8;  // 16-byte chunks per row
    const int n_slices = (hc + 63) / 64;
    const int n_blocks = (p.n_req + 15) / 16;
    uint4* tile = reinterpret_cast<uint4*>(mpart + (size_t)n_blocks * n_waves * 256) + wave * 256;
    const int row0 = blockIdx.x * 16;
    const int i = row0 / p.rank;
    const size_t row_bytes = (size_t)p.d_model * sizeof(uint16_t);
    const __amdgpu_buffer_rsrc_t a = tile_rsrc(static_cast<const char*>(p.w_down) + (size_t)row0 * row_bytes,
                                               (unsigned)(16 * row_bytes));
    // the hidden states of this indexer: requests past the batch's end lie beyond the range (the
    // stride is at least a row) and read as zeros, filling columns that are never stored
    const unsigned req_bytes = (unsigned)p.hidden_req_stride * (unsigned)sizeof(uint16_t);
    const __amdgpu_buffer_rsrc_t hb =
        tile_rsrc(static_cast<const char*>(p.hidden) + (size_t)i * p.hidden_idx_stride * sizeof(uint16_t),
                  (unsigned)(p.n_req - 1) * req_bytes + (unsigned)row_bytes);
    const unsigned lane_req = (unsigned)kc * req_bytes;
    // instruction j of quarter q of block rb: requests 16 rb + 4 j + l / 16, chunks 16 q + l % 16 of
    // the slice
    auto fetch = [&](int s, int rb, int q, uint4 (&g)[4]) {
        const int c = s * 64 + 16 * q + rl;
        const unsigned v = c < hc ? lane_req + (unsigned)c * 16u : kPastEnd;
#pragma unroll
        for (int j = 0; j < 4; ++j) g[j] = load_nt(hb, v + (unsigned)(16 * rb + 4 * j) * req_bytes, 0u);
    };
    for (int s = wave; s < n_slices; s += n_waves) {
        uint4 av[kMSteps];
#pragma unroll
        for (int t = 0; t < kMSteps; ++t) {
            const int c = s * 64 + 4 * t + kc;
            av[t] = load_nt(a, c < hc ? (unsigned)(rl * row_bytes) + (unsigned)c * 16u : kPastEnd, 0u);
        }
        uint4 g[4];
        fetch(s, 0, 0, g);
        for (int rb = 0; rb < n_blocks; ++rb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int j = 0; j < 4; ++j) tile[(4 * j + kc) * 16 + (rl ^ (4 * j + kc))] = g[j];
                __builtin_amdgcn_sched_barrier(0);  // the next loads reuse g's registers
                if (q < 3) fetch(s, rb, q + 1, g);
                else if (rb + 1 < n_blocks) fetch(s, rb + 1, 0, g);
                uint4 bv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) bv[j] = tile[rl * 16 + ((4 * j + kc) ^ rl)];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[4 * q + j]),
                                                                   __builtin_bit_cast(bf16x8, bv[j]), acc, 0, 0, 0);
            }
            // lane l holds rows 4 (l / 16) .. + 3 of request column l % 16
            float* dst = mpart + ((size_t)(rb * n_waves + wave) * 16 + 4 * kc) * 16 + rl;
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[16 * j] = s == wave ? acc[j] : dst[16 * j] + acc[j];
        }
    }
    __syncthreads();
    uint16_t* out = static_cast<uint16_t*>(p.latent);
    const int k0 = row0 - i * p.rank;
    const int w_used = min(n_waves, n_slices);
    for (int o = threadIdx.x; o < n_blocks * 256; o += blockDim.x) {
        const int rb = o / 256, e = o % 256, row = e / 16, col = e % 16;
        const int r = 16 * rb + col;
        float sum = 0.0f;
        for (int w = 0; w < w_used; ++w) sum += mpart[((size_t)(rb * n_waves + w) * 16 + row) * 16 + col];
        if (r < p.n_req) out[((size_t)r * p.n_idx + i) * p.rank + k0 + row] = Elem<uint16_t>::store(sum);
    }
}

lsa_status latent_check(const lsa_latent_args* a) {
    LSA_CHECK_ARG(a != nullptr, "lsa_query_latent: null args");
    LSA_CHECK_ARG(a->n_req >= 1 && a->n_req <= kMaxReq, "lsa_query_latent: n_req=%d outside 1..%d", a->n_req, kMaxReq);
    LSA_CHECK_SUP(dtype_ok(a->dtype), "lsa_query_latent: dtype %d", a->dtype);
    LSA_CHECK_SUP(a->d_model >= 256 && a->d_model <= 16384 && a->d_model % 256 == 0,
                  "lsa_query_latent: d_model=%d (a multiple of 256, <= 16384)", a->d_model);
    LSA_CHECK_SUP(a->rank >= 256 && a->rank <= 16384 && a->rank % 256 == 0,
                  "lsa_query_latent: rank=%d (a multiple of 256, <= 16384)", a->rank);
    LSA_CHECK_SUP(a->n_idx >= 1 && a->n_idx <= 4, "lsa_query_latent: n_idx=%d (1..4)", a->n_idx);
    LSA_CHECK_ARG(a->reserved0 == 0, "lsa_query_latent: reserved0 must be 0");
    LSA_CHECK_ARG(a->hidden && a->w_down && a->latent, "lsa_query_latent: null device pointer");
    LSA_CHECK_ARG(a->hidden_req_stride >= a->d_model || a->n_req == 1,
                  "lsa_query_latent: hidden_req_stride=%lld < d_model", (long long)a->hidden_req_stride);
    LSA_CHECK_ARG(a->hidden_idx_stride >= 0, "lsa_query_latent: negative hidden_idx_stride");
    const size_t eb = elem_bytes(a->dtype);
    LSA_CHECK_ARG(((uintptr_t)a->hidden % 16) == 0 && ((uintptr_t)a->w_down % 16) == 0 &&
                      ((uintptr_t)a->latent % 16) == 0,
                  "lsa_query_latent: hidden, w_down and latent must be 16-byte aligned");
    LSA_CHECK_ARG((a->hidden_req_stride * eb) % 16 == 0 && (a->hidden_idx_stride * eb) % 16 == 0,
                  "lsa_query_latent: hidden strides must be multiples of 16 bytes");
    return LSA_OK;
}

template <typename T>
lsa_status launch_latent(const lsa_latent_args* a, hipStream_t stream) {
    LatentParams p;
    p.hidden = a->hidden;
    p.hidden_req_stride = a->hidden_req_stride;
    p.hidden_idx_stride = a->hidden_idx_stride;
    p.w_down = a->w_down;
    p.latent = a->latent;
    p.n_req = a->n_req;
    p.d_model = a->d_model;
    p.rank = a->rank;
    p.n_idx = a->n_idx;
    const int slices = (a->d_model / Elem<T>::N + 63) / 64;
    const int waves = std::min(slices, kMaxWaves);
    const size_t req_bytes = (size_t)a->hidden_req_stride * sizeof(T);
    const size_t range = (size_t)(a->n_req - 1) * req_bytes + (size_t)a->d_model * sizeof(T);
    if (std::is_same<T, uint16_t>::value && a->n_req >= kMfmaMinReq && req_bytes < kMfmaMaxReqBytes &&
        range < kMfmaMaxRange) {
        // per wave: partial sums (1 KiB per request block) and a B tile (4 KiB); <= 64 KiB in all
        const size_t lds = ((size_t)((a->n_req + 15) / 16) * 256 * sizeof(float) + 256 * sizeof(uint4)) * waves;
        const dim3 grid(a->n_idx * a->rank / 16), block(64 * waves);
        if (a->ev_begin && a->ev_end)
            hipExtLaunchKernelGGL(latent_mfma_kernel, grid, block, lds, stream, a->ev_begin, a->ev_end, 0, p);
        else
            hipLaunchKernelGGL(latent_mfma_kernel, grid, block, lds, stream, p);
        LSA_HIP(hipGetLastError());
        return LSA_OK;
    }
    const size_t lds = (size_t)((a->n_req + kQ - 1) / kQ) * waves * kN * sizeof(float);  // <= 32 KiB
    const dim3 grid(a->n_idx * a->rank / kG), block(64 * waves);
    if (a->ev_begin && a->ev_end)  // the events take the dispatch's own start and end timestamps
        hipExtLaunchKernelGGL(latent_kernel<T>, grid, block, lds, stream, a->ev_begin, a->ev_end, 0, p);
    else
        hipLaunchKernelGGL(latent_kernel<T>, grid, block, lds, stream, p);
    LSA_HIP(hipGetLastError());
    return LSA_OK;
}

}  // namespace
}  // namespace lsa

using namespace lsa;

extern "C" lsa_status lsa_query_latent(const lsa_latent_args* a, hipStream_t stream) {
    lsa_status st = latent_check(a);
    if (st != LSA_OK) return st;
    if (a->dtype == LSA_BF16) return launch_latent<uint16_t>(a, stream);
    return launch_latent<float>(a, stream);
}
