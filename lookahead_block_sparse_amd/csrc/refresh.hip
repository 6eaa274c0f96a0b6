// Index refresh: Query Encoder, dual-encoder block logits, sigmoid>0.5 threshold, OR-union and
// ordered compaction of the loaded-block list (zhichai.net explainer of "FlashMemory-DeepSeek-V4",
// section 2 steps 2-3, section 3 (Query Encoder, frozen KIComp keys), section 4 (OR-mode union)).
//
// Two kernels on the caller's stream:
//   encode_kernel  q[r][i][j] = sum_m W_q[i][j][m] h[r][i][m]; one wave per output row (i, j), the
//                  W_q row is read once for all requests of the call; fp32 accumulation, q stays fp32.
//   score_kernel   one work-group per 64-block word of one request, one wave per indexer.  Each wave
//                  streams its 64 key rows (8 lanes per row, 16-byte loads), forms z = q.k + bias in
//                  fp32, and turns z > 0 into a 64-bit word with a wavefront ballot.  The group ORs the
//                  indexer words.  The last group of a request (atomic ticket) scans the request's word
//                  popcounts and writes the ascending block ids and the count.
#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int kMaxReq = LSA_MAX_REFRESH_REQ;

struct EncodeParams {
    const void* hidden;
    long long hidden_req_stride, hidden_idx_stride;
    const void* w_q;
    float* q;              // [n_req][n_idx][d_idx]
    unsigned* tickets;     // [n_req], zeroed here for the score kernel
    int n_req, d_model, d_idx, n_idx;
};

struct ScoreParams {
    const void* keys;
    const float* q;
    const float* bias;
    int* sel_ids;
    int* sel_count;
    unsigned long long* masks;
    unsigned long long* words;  // [total_words] union words (workspace)
    unsigned* tickets;
    int n_req, n_idx;
    long long blk_off[kMaxReq + 1];
    int word_off[kMaxReq + 1];
};

// 16 bytes of T: 8 bf16 or 4 fp32, dotted with the matching fp32 values.
template <typename T>
struct Chunk;

template <>
struct Chunk<uint16_t> {
    static constexpr int N = 8;
    __device__ static float dot(uint4 w, const float* x) {
        float a = bf16_lo(w.x) * x[0];
        a = fmaf(bf16_hi(w.x), x[1], a);
        a = fmaf(bf16_lo(w.y), x[2], a);
        a = fmaf(bf16_hi(w.y), x[3], a);
        a = fmaf(bf16_lo(w.z), x[4], a);
        a = fmaf(bf16_hi(w.z), x[5], a);
        a = fmaf(bf16_lo(w.w), x[6], a);
        a = fmaf(bf16_hi(w.w), x[7], a);
        return a;
    }
    __device__ static void widen(uint4 w, float* x) {
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
        x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
    }
};

template <>
struct Chunk<float> {
    static constexpr int N = 4;
    __device__ static float dot(uint4 w, const float* x) {
        float a = __uint_as_float(w.x) * x[0];
        a = fmaf(__uint_as_float(w.y), x[1], a);
        a = fmaf(__uint_as_float(w.z), x[2], a);
        a = fmaf(__uint_as_float(w.w), x[3], a);
        return a;
    }
    __device__ static void widen(uint4 w, float* x) {
        x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
    }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// ------------------------------------------------------------------------------------------
// Query Encoder.  Grid: ceil(n_idx*d_idx/4) groups of 256 threads; wave w of group g owns output row
// 4g+w.  Lane l reads 16-byte chunks l, l+64, ... of the W_q row and of each request's hidden state.
template <typename T>
__global__ __launch_bounds__(256) void encode_kernel(EncodeParams p) {
    using C = Chunk<T>;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (blockIdx.x == 0 && threadIdx.x < p.n_req) p.tickets[threadIdx.x] = 0u;
    if (row >= p.n_idx * p.d_idx) return;
    const int i = row / p.d_idx;
    const int n_chunks = p.d_model / C::N;  // 16-byte chunks per row
    const uint4* w = reinterpret_cast<const uint4*>(static_cast<const T*>(p.w_q) + (size_t)row * p.d_model);
    const T* hid = static_cast<const T*>(p.hidden) + (size_t)i * p.hidden_idx_stride;

    for (int r0 = 0; r0 < p.n_req; r0 += 8) {
        float acc[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) acc[rr] = 0.f;
        for (int c0 = 0; c0 < n_chunks; c0 += 64 * 8) {
            uint4 wc[8];
            float wf[8][C::N];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int c = c0 + k * 64 + lane;
                wc[k] = c < n_chunks ? w[c] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) C::widen(wc[k], wf[k]);
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                if (r0 + rr >= p.n_req) break;
                const uint4* h = reinterpret_cast<const uint4*>(hid + (size_t)(r0 + rr) * p.hidden_req_stride);
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int c = c0 + k * 64 + lane;
                    if (c < n_chunks) acc[rr] += C::dot(h[c], wf[k]);
                }
            }
        }
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            if (r0 + rr >= p.n_req) break;
            const float s = wave_sum(acc[rr]);
            if (lane == 0) p.q[(size_t)(r0 + rr) * p.n_idx * p.d_idx + row] = s;
        }
    }
}

// ------------------------------------------------------------------------------------------
// Scoring + threshold + union + compaction.  Grid: one group per word (64 blocks) over all requests;
// blockDim = 64 * n_idx (wave i = indexer i).
template <typename T, int DIDX>
__global__ __launch_bounds__(256) void score_kernel(ScoreParams p) {
    using C = Chunk<T>;
    constexpr int ROW_BYTES = DIDX * (int)sizeof(T);
    constexpr int LPR = ROW_BYTES / 128;        // 16-byte loads per lane per row (8 lanes per row)
    constexpr int QPL = LPR * C::N;             // q values held per lane
    static_assert(LPR >= 1 && LPR <= 8, "row size");

    __shared__ unsigned long long s_words[4];
    __shared__ int s_last;
    __shared__ int s_scan[256];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int word = blockIdx.x;

    // request of this word (uniform)
    int r = 0;
    while (r + 1 < p.n_req && p.word_off[r + 1] <= word) ++r;
    const int lw = word - p.word_off[r];
    const long long b_first = p.blk_off[r];
    const int n_blk = (int)(p.blk_off[r + 1] - b_first);
    const int b0 = lw * 64;
    const int n_valid = min(64, n_blk - b0);
    const int n_words_r = p.word_off[r + 1] - p.word_off[r];

    // ---- one indexer per wave ----
    {
        const int i = wave;
        const int x = lane & 7;        // 16-byte column within a 128-byte slice of the row
        const int rsub = lane >> 3;    // row within a group of 8 rows
        const float* qv = p.q + ((size_t)r * p.n_idx + i) * DIDX;
        float qr[QPL];
#pragma unroll
        for (int k = 0; k < LPR; ++k) {
#pragma unroll
            for (int e = 0; e < C::N; ++e) qr[k * C::N + e] = qv[(k * 128 + x * 16) / (int)sizeof(T) + e];
        }
        const float bias = p.bias[r * p.n_idx + i];
        const char* rows = static_cast<const char*>(p.keys) +
                           ((size_t)p.n_idx * b_first + (size_t)i * n_blk + b0) * ROW_BYTES;

        constexpr int GROUPS = 8;            // 8 rows per group, 8 groups = 64 rows
        constexpr int HALF = (LPR == 8) ? 2 : 1;
        unsigned long long bits = 0ull;
#pragma unroll
        for (int hh = 0; hh < HALF; ++hh) {
            constexpr int GH = GROUPS / HALF;
            uint4 v[GH][LPR];
#pragma unroll
            for (int g = 0; g < GH; ++g) {
                const int rowi = (hh * GH + g) * 8 + rsub;
                const bool ok = rowi < n_valid;
                const uint4* src = reinterpret_cast<const uint4*>(rows + (size_t)rowi * ROW_BYTES + x * 16);
#pragma unroll
                for (int k = 0; k < LPR; ++k) v[g][k] = ok ? src[k * 8] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int g = 0; g < GH; ++g) {
                const int rowi = (hh * GH + g) * 8 + rsub;
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < LPR; ++k) acc += C::dot(v[g][k], qr + k * C::N);
                acc += __shfl_xor(acc, 1, 64);
                acc += __shfl_xor(acc, 2, 64);
                acc += __shfl_xor(acc, 4, 64);
                const bool keep = (rowi < n_valid) && (acc + bias > 0.f);
                const unsigned long long m = __ballot(keep);
                // lanes 8j..8j+7 all hold row 8g'+j; take bit 8j
                unsigned long long b8 = 0ull;
#pragma unroll
                for (int j = 0; j < 8; ++j) b8 |= ((m >> (8 * j)) & 1ull) << j;
                bits |= b8 << (8 * (hh * GH + g));
            }
        }
        if (lane == 0) s_words[i] = bits;
        if (p.masks && lane == 0) {
            const size_t base = (size_t)(p.n_idx + 1) * p.word_off[r];
            p.masks[base + (size_t)i * n_words_r + lw] = bits;
        }
    }
    __syncthreads();

    // ---- union + ticket ----
    if (threadIdx.x == 0) {
        unsigned long long u = 0ull;
        for (int i = 0; i < p.n_idx; ++i) u |= s_words[i];
        if (p.masks) {
            const size_t base = (size_t)(p.n_idx + 1) * p.word_off[r];
            p.masks[base + (size_t)p.n_idx * n_words_r + lw] = u;
        }
        __hip_atomic_store(&p.words[word], u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __threadfence();
        const unsigned t = atomicAdd(&p.tickets[r], 1u);
        s_last = (t == (unsigned)(n_words_r - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;

    // ---- the last group of request r compacts its words into ascending ids ----
    __threadfence();
    const int nt = blockDim.x;
    const int per = (n_words_r + nt - 1) / nt;  // consecutive words per thread
    const int w0 = min(n_words_r, (int)threadIdx.x * per);
    const int w1 = min(n_words_r, w0 + per);
    const unsigned long long* words_r = p.words + p.word_off[r];
    int cnt = 0;
    for (int w = w0; w < w1; ++w)
        cnt += __popcll(__hip_atomic_load(&words_r[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    // block-wide exclusive scan of cnt
    s_scan[threadIdx.x] = cnt;
    __syncthreads();
    for (int off = 1; off < nt; off <<= 1) {
        const int v = threadIdx.x >= (unsigned)off ? s_scan[threadIdx.x - off] : 0;
        __syncthreads();
        s_scan[threadIdx.x] += v;
        __syncthreads();
    }
    int pos = s_scan[threadIdx.x] - cnt;
    int* out = p.sel_ids + b_first;
    for (int w = w0; w < w1; ++w) {
        unsigned long long u = __hip_atomic_load(&words_r[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        while (u) {
            const int bit = __ffsll((long long)u) - 1;
            out[pos++] = w * 64 + bit;
            u &= u - 1;
        }
    }
    if (threadIdx.x == nt - 1) p.sel_count[r] = s_scan[nt - 1];
}

struct RefreshLayout {
    size_t q_off, words_off, tickets_off, total;
    int total_words;
};

lsa_status refresh_layout(const lsa_refresh_args* a, RefreshLayout* L) {
    LSA_CHECK_ARG(a != nullptr, "lsa_index_refresh: null args");
    LSA_CHECK_ARG(a->n_req >= 1 && a->n_req <= kMaxReq, "lsa_index_refresh: n_req=%d outside 1..%d",
                  a->n_req, kMaxReq);
    LSA_CHECK_SUP(dtype_ok(a->dtype), "lsa_index_refresh: dtype %d", a->dtype);
    LSA_CHECK_SUP(a->d_idx == 128 || a->d_idx == 256, "lsa_index_refresh: d_idx=%d (128 or 256)", a->d_idx);
    LSA_CHECK_SUP(a->n_idx >= 1 && a->n_idx <= 4, "lsa_index_refresh: n_idx=%d (1..4)", a->n_idx);
    LSA_CHECK_SUP(a->d_model >= 256 && a->d_model % 256 == 0 && a->d_model <= 16384,
                  "lsa_index_refresh: d_model=%d (multiple of 256, <= 16384)", a->d_model);
    LSA_CHECK_ARG(a->reserved0 == 0, "lsa_index_refresh: reserved0 must be 0");
    LSA_CHECK_ARG(a->blk_off != nullptr, "lsa_index_refresh: blk_off is null");
    LSA_CHECK_ARG(a->blk_off[0] == 0, "lsa_index_refresh: blk_off[0] must be 0");
    long long words = 0;
    for (int r = 0; r < a->n_req; ++r) {
        const long long nb = a->blk_off[r + 1] - a->blk_off[r];
        LSA_CHECK_ARG(nb >= 1 && nb <= (1ll << 24), "lsa_index_refresh: request %d has %lld blocks", r, nb);
        words += (nb + 63) / 64;
    }
    LSA_CHECK_ARG(words <= (1ll << 30), "lsa_index_refresh: too many blocks");
    L->total_words = (int)words;
    size_t off = 0;
    L->q_off = off;
    off = align_up(off + (size_t)a->n_req * a->n_idx * a->d_idx * sizeof(float), 256);
    L->words_off = off;
    off = align_up(off + (size_t)words * sizeof(unsigned long long), 256);
    L->tickets_off = off;
    off = align_up(off + (size_t)a->n_req * sizeof(unsigned), 256);
    L->total = off;
    return LSA_OK;
}

template <typename T>
lsa_status launch_refresh(const lsa_refresh_args* a, const RefreshLayout& L, hipStream_t stream) {
    char* ws = static_cast<char*>(a->workspace);
    EncodeParams ep{};
    ep.hidden = a->hidden;
    ep.hidden_req_stride = a->hidden_req_stride;
    ep.hidden_idx_stride = a->hidden_idx_stride;
    ep.w_q = a->w_q;
    ep.q = reinterpret_cast<float*>(ws + L.q_off);
    ep.tickets = reinterpret_cast<unsigned*>(ws + L.tickets_off);
    ep.n_req = a->n_req;
    ep.d_model = a->d_model;
    ep.d_idx = a->d_idx;
    ep.n_idx = a->n_idx;
    const int rows = a->n_idx * a->d_idx;
    hipLaunchKernelGGL(encode_kernel<T>, dim3((rows + 3) / 4), dim3(256), 0, stream, ep);
    LSA_HIP(hipGetLastError());

    ScoreParams sp{};
    sp.keys = a->keys;
    sp.q = ep.q;
    sp.bias = a->bias;
    sp.sel_ids = a->sel_ids;
    sp.sel_count = a->sel_count;
    sp.masks = reinterpret_cast<unsigned long long*>(a->masks);
    sp.words = reinterpret_cast<unsigned long long*>(ws + L.words_off);
    sp.tickets = ep.tickets;
    sp.n_req = a->n_req;
    sp.n_idx = a->n_idx;
    int wo = 0;
    for (int r = 0; r <= a->n_req; ++r) {
        sp.blk_off[r] = a->blk_off[r];
        sp.word_off[r] = wo;
        if (r < a->n_req) wo += (int)((a->blk_off[r + 1] - a->blk_off[r] + 63) / 64);
    }
    const dim3 grid(L.total_words), block(64 * a->n_idx);
    if (a->d_idx == 256)
        hipLaunchKernelGGL((score_kernel<T, 256>), grid, block, 0, stream, sp);
    else
        hipLaunchKernelGGL((score_kernel<T, 128>), grid, block, 0, stream, sp);
    LSA_HIP(hipGetLastError());
    return LSA_OK;
}

}  // namespace
}  // namespace lsa

using namespace lsa;

extern "C" lsa_status lsa_index_refresh_workspace(const lsa_refresh_args* a, size_t* bytes) {
    RefreshLayout L;
    lsa_status st = refresh_layout(a, &L);
    if (st != LSA_OK) return st;
    LSA_CHECK_ARG(bytes != nullptr, "lsa_index_refresh_workspace: bytes is null");
    *bytes = L.total;
    return LSA_OK;
}

extern "C" lsa_status lsa_index_refresh(const lsa_refresh_args* a, hipStream_t stream) {
    RefreshLayout L;
    lsa_status st = refresh_layout(a, &L);
    if (st != LSA_OK) return st;
    LSA_CHECK_ARG(a->hidden && a->w_q && a->keys && a->bias && a->sel_ids && a->sel_count,
                  "lsa_index_refresh: null device pointer");
    LSA_CHECK_ARG(a->hidden_req_stride >= a->d_model || a->n_req == 1,
                  "lsa_index_refresh: hidden_req_stride=%lld < d_model", (long long)a->hidden_req_stride);
    LSA_CHECK_ARG(a->hidden_idx_stride >= 0, "lsa_index_refresh: negative hidden_idx_stride");
    if (a->workspace == nullptr || a->workspace_bytes < L.total)
        return fail(LSA_ERR_WORKSPACE, "lsa_index_refresh: workspace of %zu bytes, need %zu",
                    a->workspace ? a->workspace_bytes : (size_t)0, L.total);
    // 16-byte loads need 16-byte aligned rows
    const size_t eb = elem_bytes(a->dtype);
    LSA_CHECK_ARG(((uintptr_t)a->hidden % 16) == 0 && ((uintptr_t)a->w_q % 16) == 0 &&
                      ((uintptr_t)a->keys % 16) == 0 && ((uintptr_t)a->workspace % 16) == 0,
                  "lsa_index_refresh: hidden, w_q, keys and workspace must be 16-byte aligned");
    LSA_CHECK_ARG((a->hidden_req_stride * eb) % 16 == 0 && (a->hidden_idx_stride * eb) % 16 == 0,
                  "lsa_index_refresh: hidden strides must be multiples of 16 bytes");
    if (a->dtype == LSA_BF16) return launch_refresh<uint16_t>(a, L, stream);
    return launch_refresh<float>(a, L, stream);
}
