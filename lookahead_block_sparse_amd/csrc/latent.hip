// Low-rank query projection, first factor: the latent c_i = A_i h of every indexer (zhichai.net
// explainer of "FlashMemory-DeepSeek-V4", section 4, training tricks: a query projection of rank
// 2048 through the backbone's MLA/MQA bottleneck).  The refresh's Query Encoder then projects the
// latent with B_i.
//
// A GEMV over A [n_idx][rank][d_model] shared by every request, HBM-bound on A (25 M elements at
// n_idx = 3, r = 2048, d = 4096): each wave owns kRows rows of A and reads each row once for every
// request; lane l reads 16-byte chunks l, l+64, ... of the row; fp32 accumulation, a wavefront sum,
// and the latent stored in the input type (bf16: round to nearest, ties to even).
#include <hip/hip_ext.h>

#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int kMaxReq = LSA_MAX_REFRESH_REQ;
constexpr int kThreads = 256;
constexpr int kRows = 2;  // rows of A per wave
constexpr int kReq = 4;   // requests per round

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// A is read once per call: non-temporal 16-byte loads
__device__ __forceinline__ uint4 load_nt(const uint4* q) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q));
    return make_uint4(v.x, v.y, v.z, v.w);
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
    // acc + a.b over 8 bf16 pairs with the packed dot of two bf16 pairs into fp32
    // (v_dot2_f32_bf16: the products of bf16 values are exact in fp32), 4 instructions where
    // unpacking both operands and fusing would take 24 (the unpacking made the kernel ALU-bound)
    __device__ static float dot_acc(uint4 a, uint4 b, float acc) {
        acc = __builtin_amdgcn_fdot2_f32_bf16(bf2(a.x), bf2(b.x), acc, false);
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
    __device__ static float dot_acc(uint4 a, uint4 b, float acc) {
        acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
        acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
        acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
        return fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
    }
    __device__ static float store(float x) { return x; }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void latent_kernel(LatentParams p) {
    using E = Elem<T>;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * (kThreads / 64) + wave) * kRows;  // over n_idx * rank rows
    const int n_rows = p.n_idx * p.rank;
    if (row0 >= n_rows) return;
    const int i = row0 / p.rank;  // rank is a multiple of kRows: a wave's rows share the indexer
    const int hc = p.d_model / E::N;  // 16-byte chunks per row
    const uint4* a = reinterpret_cast<const uint4*>(static_cast<const T*>(p.w_down) + (size_t)row0 * p.d_model);
    const T* hid = static_cast<const T*>(p.hidden) + (size_t)i * p.hidden_idx_stride;
    T* out = static_cast<T*>(p.latent);
    for (int r0 = 0; r0 < p.n_req; r0 += kReq) {
        float acc[kRows][kReq] = {};
        for (int c0 = 0; c0 < hc; c0 += 64 * 4) {
            // unconditional loads from clamped indices (masked after loading) keep all in flight
            uint4 wc[kRows][4];
            uint4 hv[kReq][4];
#pragma unroll
            for (int jj = 0; jj < kRows; ++jj)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    wc[jj][k] = load_nt(a + (size_t)jj * hc + min(c0 + k * 64 + lane, hc - 1));
#pragma unroll
            for (int rr = 0; rr < kReq; ++rr) {
                const uint4* h = reinterpret_cast<const uint4*>(hid + (size_t)min(r0 + rr, p.n_req - 1) * p.hidden_req_stride);
#pragma unroll
                for (int k = 0; k < 4; ++k) hv[rr][k] = h[min(c0 + k * 64 + lane, hc - 1)];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool live = c0 + k * 64 + lane < hc;
#pragma unroll
                for (int jj = 0; jj < kRows; ++jj)
#pragma unroll
                    for (int rr = 0; rr < kReq; ++rr) {
                        const float t = E::dot_acc(wc[jj][k], hv[rr][k], acc[jj][rr]);
                        acc[jj][rr] = live ? t : acc[jj][rr];
                    }
            }
        }
#pragma unroll
        for (int jj = 0; jj < kRows; ++jj)
#pragma unroll
            for (int rr = 0; rr < kReq; ++rr) {
                float v = acc[jj][rr];
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
                if (lane == jj * kReq + rr && r0 + rr < p.n_req) {
                    const int k = row0 + jj - i * p.rank;
                    out[((size_t)(r0 + rr) * p.n_idx + i) * p.rank + k] = E::store(v);
                }
            }
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
    const int rows_per_group = kRows * (kThreads / 64);
    const dim3 grid((a->n_idx * a->rank + rows_per_group - 1) / rows_per_group), block(kThreads);
    if (a->ev_begin && a->ev_end)  // the events take the dispatch's own start and end timestamps
        hipExtLaunchKernelGGL(latent_kernel<T>, grid, block, 0, stream, a->ev_begin, a->ev_end, 0, p);
    else
        hipLaunchKernelGGL(latent_kernel<T>, grid, block, 0, stream, p);
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
