// Index refresh: Query Encoder, dual-encoder block logits, sigmoid>0.5 threshold, OR-union and
// ordered compaction of the loaded-block list (zhichai.net explainer of "FlashMemory-DeepSeek-V4",
// section 2 steps 2-3, section 3 (Query Encoder, frozen KIComp keys), section 4 (OR-mode union)).
//
// Two kernels on the caller's stream:
//   encode_kernel  q[r][i][j] = sum_m W_q[i][j][m] h[r][i][m]: one wave per output row (i, j), the row
//                  read once for every request of the call, fp32 accumulation, q kept in fp32.  It also
//                  clears the score kernel's per-request counters and word slots.
//   score_kernel   one group per 64-block word of one request, two waves per indexer.  Each wave issues
//                  all loads of its 32 key rows at once (8 lanes per row, 16-byte loads), forms
//                  z = q.k + bias in fp32 and turns z > 0 into a 64-bit word with a wavefront ballot;
//                  the group ORs the indexer words into the union word.  The group publishes the union
//                  word and counts itself on its request's counter; the group that counts last scans the
//                  request's word popcounts and writes the ascending ids and the count.  Groups never wait
//                  for each other: the last one only reads words whose writers have all finished.
// Cross-group values travel in 64-bit words written with device-scope atomic stores and carrying a
// "written" flag, read with device-scope atomic loads, so no memory fence is needed.  Atomics on one
// address serialize on this GPU, hence one counter per request instead of one for the whole launch.
#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int kMaxReq = LSA_MAX_REFRESH_REQ;
constexpr unsigned kSpinLimit = 1u << 16;
constexpr unsigned long long kWritten = 1ull << 32;

struct EncodeParams {
    const void* hidden;
    long long hidden_req_stride, hidden_idx_stride;
    const void* w_q;
    float* q;                         // [n_req][n_idx][d_idx]
    unsigned* counters;               // [n_req], cleared here
    unsigned long long* words;        // [total_words][2], cleared here
    int n_req, d_model, d_idx, n_idx, total_words;
};

struct ScoreParams {
    const void* keys;
    const float* q;
    const float* bias;
    int* sel_ids;
    int* sel_count;
    unsigned long long* masks;
    unsigned long long* words;  // [total_words][2]: union word halves, each (written flag << 32 | 32 bits)
    unsigned* counters;
    int n_req, n_idx;
    long long blk_off[kMaxReq + 1];
    int word_off[kMaxReq + 1];
};

// 16 bytes of T: 8 bf16 or 4 fp32.
template <typename T>
struct Chunk;

template <>
struct Chunk<uint16_t> {
    static constexpr int N = 8;
    __device__ static void widen(uint4 w, float* x) {
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
        x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
    }
};

template <>
struct Chunk<float> {
    static constexpr int N = 4;
    __device__ static void widen(uint4 w, float* x) {
        x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
        x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
    }
};

template <typename T>
__device__ __forceinline__ float dot_chunks(uint4 a, uint4 b) {
    float x[Chunk<T>::N], y[Chunk<T>::N];
    Chunk<T>::widen(a, x);
    Chunk<T>::widen(b, y);
    float s = x[0] * y[0];
#pragma unroll
    for (int e = 1; e < Chunk<T>::N; ++e) s = fmaf(x[e], y[e], s);
    return s;
}

template <typename T>
__device__ __forceinline__ float dot_chunk_f32(uint4 a, const float* y) {
    float x[Chunk<T>::N];
    Chunk<T>::widen(a, x);
    float s = x[0] * y[0];
#pragma unroll
    for (int e = 1; e < Chunk<T>::N; ++e) s = fmaf(x[e], y[e], s);
    return s;
}

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
    if (blockIdx.x == 0) {
        for (int e = threadIdx.x; e < p.n_req; e += 256) p.counters[e] = 0u;
    }
    for (int e = blockIdx.x * 256 + threadIdx.x; e < 2 * p.total_words; e += gridDim.x * 256) p.words[e] = 0ull;
    if (row >= p.n_idx * p.d_idx) return;
    const int i = row / p.d_idx;
    const int n_chunks = p.d_model / C::N;
    const uint4* w = reinterpret_cast<const uint4*>(static_cast<const T*>(p.w_q) + (size_t)row * p.d_model);
    const T* hid = static_cast<const T*>(p.hidden) + (size_t)i * p.hidden_idx_stride;
    for (int r0 = 0; r0 < p.n_req; r0 += 4) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < n_chunks; c0 += 64 * 8) {
            // unconditional loads from clamped indices (zeroed after loading) keep all in flight
            uint4 wc[8];
            uint4 hc[4][8];
#pragma unroll
            for (int k = 0; k < 8; ++k) wc[k] = w[min(c0 + k * 64 + lane, n_chunks - 1)];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const uint4* h = reinterpret_cast<const uint4*>(hid + (size_t)min(r0 + rr, p.n_req - 1) * p.hidden_req_stride);
#pragma unroll
                for (int k = 0; k < 8; ++k) hc[rr][k] = h[min(c0 + k * 64 + lane, n_chunks - 1)];
            }
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float d = dot_chunks<T>(wc[k], hc[rr][k]);
                    acc[rr] += (c0 + k * 64 + lane < n_chunks) ? d : 0.f;
                }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const float s = wave_sum(acc[rr]);
            if (lane == 0 && r0 + rr < p.n_req) p.q[(size_t)(r0 + rr) * p.n_idx * p.d_idx + row] = s;
        }
    }
}

// ------------------------------------------------------------------------------------------
// Scoring + threshold + union + compaction.  Grid: one group per word (64 blocks) over all requests;
// blockDim = 128 * n_idx: waves 2i and 2i+1 score rows 0..31 and 32..63 of indexer i.
constexpr int kScoreWavesPerIdx = 2;

template <typename T, int DIDX>
__global__ __launch_bounds__(128 * 4, 3) void score_kernel(ScoreParams p) {
    using C = Chunk<T>;
    constexpr int ROW_BYTES = DIDX * (int)sizeof(T);
    constexpr int LPR = ROW_BYTES / 128;  // 16-byte loads per lane per row (8 lanes per row)
    constexpr int QPL = LPR * C::N;       // q values held per lane
    constexpr int HALF = (LPR == 8) ? 2 : 1;
    constexpr int GH = 4 / HALF;          // groups of 8 rows per pass (32 rows per wave)
    static_assert(LPR >= 1 && LPR <= 8, "row size");

    __shared__ unsigned s_half[8];
    __shared__ int s_last;
    __shared__ int s_scan[512];
    __shared__ unsigned s_missing;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int word = blockIdx.x;
    int r = 0;
    while (r + 1 < p.n_req && p.word_off[r + 1] <= word) ++r;
    const int lw = word - p.word_off[r];
    const long long b_first = p.blk_off[r];
    const int n_blk = (int)(p.blk_off[r + 1] - b_first);
    const int b0 = lw * 64;
    const int n_valid = min(64, n_blk - b0);
    const int n_words_r = p.word_off[r + 1] - p.word_off[r];

    // ---- 32 rows of one indexer per wave ----
    {
        const int i = wave / kScoreWavesPerIdx;
        const int half = wave % kScoreWavesPerIdx;
        const int x = lane & 7;      // 16-byte column inside a 128-byte slice of the row
        const int rsub = lane >> 3;  // row inside a group of 8 rows
        const char* rows = static_cast<const char*>(p.keys) + ((size_t)p.n_idx * b_first + (size_t)i * n_blk + b0) * ROW_BYTES;
        const float* qv = p.q + ((size_t)r * p.n_idx + i) * DIDX;
        const float bias = p.bias[r * p.n_idx + i];
        unsigned bits = 0u;
#pragma unroll
        for (int hh = 0; hh < HALF; ++hh) {
            // unconditional loads (rows past the request's last block re-read its last row and are
            // masked out below), so all of them are in flight together
            uint4 v[GH][LPR];
#pragma unroll
            for (int g = 0; g < GH; ++g) {
                const int rowi = min(32 * half + (hh * GH + g) * 8 + rsub, n_valid - 1);
                const uint4* src = reinterpret_cast<const uint4*>(rows + (size_t)rowi * ROW_BYTES + x * 16);
#pragma unroll
                for (int k = 0; k < LPR; ++k) v[g][k] = src[k * 8];
            }
            float qr[QPL];
#pragma unroll
            for (int k = 0; k < LPR; ++k)
#pragma unroll
                for (int e = 0; e < C::N; ++e) qr[k * C::N + e] = qv[(k * 128 + x * 16) / (int)sizeof(T) + e];
#pragma unroll
            for (int g = 0; g < GH; ++g) {
                const int rowi = 32 * half + (hh * GH + g) * 8 + rsub;
                float acc = 0.f;
#pragma unroll
                for (int k = 0; k < LPR; ++k) acc += dot_chunk_f32<T>(v[g][k], qr + k * C::N);
                acc += __shfl_xor(acc, 1, 64);
                acc += __shfl_xor(acc, 2, 64);
                acc += __shfl_xor(acc, 4, 64);
                const bool keep = (rowi < n_valid) && (acc + bias > 0.f);
                const unsigned long long m = __ballot(keep);
                unsigned b8 = 0u;  // lanes 8j..8j+7 all hold row 8g+j: take bit 8j
#pragma unroll
                for (int j = 0; j < 8; ++j) b8 |= (unsigned)((m >> (8 * j)) & 1ull) << j;
                bits |= b8 << (8 * (hh * GH + g));
            }
        }
        if (lane == 0) s_half[wave] = bits;
    }
    __syncthreads();
    if (p.masks && threadIdx.x < p.n_idx) {
        const int i = threadIdx.x;
        const unsigned long long w64 = (unsigned long long)s_half[2 * i] | ((unsigned long long)s_half[2 * i + 1] << 32);
        p.masks[(size_t)(p.n_idx + 1) * p.word_off[r] + (size_t)i * n_words_r + lw] = w64;
    }

    // ---- union word, published; count this group on its request ----
    if (threadIdx.x == 0) {
        unsigned long long u = 0ull;
        for (int i = 0; i < p.n_idx; ++i)
            u |= (unsigned long long)s_half[2 * i] | ((unsigned long long)s_half[2 * i + 1] << 32);
        if (p.masks) p.masks[(size_t)(p.n_idx + 1) * p.word_off[r] + (size_t)p.n_idx * n_words_r + lw] = u;
        __hip_atomic_store(&p.words[2 * word], kWritten | (u & 0xffffffffull), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&p.words[2 * word + 1], kWritten | (u >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);  // both halves stored before the count is taken
        const unsigned t = atomicAdd(&p.counters[r], 1u);
        s_last = (t == (unsigned)(n_words_r - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;

    // ---- the last group of request r: scan the word popcounts, write ascending ids ----
    const int nt = blockDim.x;
    const int per = (n_words_r + nt - 1) / nt;  // consecutive words per thread
    const int w0 = min(n_words_r, (int)threadIdx.x * per);
    const int w1 = min(n_words_r, w0 + per);
    const unsigned long long* words_r = p.words + 2 * (size_t)p.word_off[r];
    auto read_word = [&](int w, bool* ok) -> unsigned long long {
        const unsigned long long lo = __hip_atomic_load(&words_r[2 * w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long hi = __hip_atomic_load(&words_r[2 * w + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *ok = (lo & kWritten) && (hi & kWritten);
        return (lo & 0xffffffffull) | (hi << 32);
    };
    // every writer counted itself after storing, so the flags are set; check them anyway (bounded)
    for (unsigned spins = 0;; ++spins) {
        if (threadIdx.x == 0) s_missing = 0u;
        __syncthreads();
        for (int w = w0; w < w1; ++w) {
            bool ok;
            read_word(w, &ok);
            if (!ok) s_missing = 1u;
        }
        __syncthreads();
        if (!s_missing || spins > kSpinLimit) break;
        __builtin_amdgcn_s_sleep(2);
    }
    int cnt = 0;
    for (int w = w0; w < w1; ++w) {
        bool ok;
        cnt += __popcll(read_word(w, &ok));
    }
    s_scan[threadIdx.x] = cnt;
    __syncthreads();
    for (int off = 1; off < nt; off <<= 1) {
        const int v = (int)threadIdx.x >= off ? s_scan[threadIdx.x - off] : 0;
        __syncthreads();
        s_scan[threadIdx.x] += v;
        __syncthreads();
    }
    int pos = s_scan[threadIdx.x] - cnt;
    int* out = p.sel_ids + b_first;
    for (int w = w0; w < w1; ++w) {
        bool ok;
        unsigned long long u = read_word(w, &ok);
        while (u) {
            const int bit = __ffsll((long long)u) - 1;
            out[pos++] = w * 64 + bit;
            u &= u - 1;
        }
    }
    if (threadIdx.x == nt - 1) p.sel_count[r] = s_missing ? -1 : s_scan[nt - 1];
}

struct RefreshLayout {
    size_t q_off, words_off, counters_off, total;
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
    LSA_CHECK_ARG(words <= (1ll << 28), "lsa_index_refresh: too many blocks");
    L->total_words = (int)words;
    size_t off = 0;
    L->q_off = off;
    off = align_up(off + (size_t)a->n_req * a->n_idx * a->d_idx * sizeof(float), 256);
    L->words_off = off;
    off = align_up(off + (size_t)words * 2 * sizeof(unsigned long long), 256);
    L->counters_off = off;
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
    ep.counters = reinterpret_cast<unsigned*>(ws + L.counters_off);
    ep.words = reinterpret_cast<unsigned long long*>(ws + L.words_off);
    ep.n_req = a->n_req;
    ep.d_model = a->d_model;
    ep.d_idx = a->d_idx;
    ep.n_idx = a->n_idx;
    ep.total_words = L.total_words;
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
    sp.words = ep.words;
    sp.counters = ep.counters;
    sp.n_req = a->n_req;
    sp.n_idx = a->n_idx;
    int wo = 0;
    for (int r = 0; r <= a->n_req; ++r) {
        sp.blk_off[r] = a->blk_off[r];
        sp.word_off[r] = wo;
        if (r < a->n_req) wo += (int)((a->blk_off[r + 1] - a->blk_off[r] + 63) / 64);
    }
    const dim3 grid(L.total_words), block(64 * kScoreWavesPerIdx * a->n_idx);
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
    const size_t eb = elem_bytes(a->dtype);
    LSA_CHECK_ARG(((uintptr_t)a->hidden % 16) == 0 && ((uintptr_t)a->w_q % 16) == 0 &&
                      ((uintptr_t)a->keys % 16) == 0 && ((uintptr_t)a->workspace % 256) == 0,
                  "lsa_index_refresh: hidden, w_q, keys must be 16-byte aligned and workspace 256-byte aligned");
    LSA_CHECK_ARG((a->hidden_req_stride * eb) % 16 == 0 && (a->hidden_idx_stride * eb) % 16 == 0,
                  "lsa_index_refresh: hidden strides must be multiples of 16 bytes");
    if (a->dtype == LSA_BF16) return launch_refresh<uint16_t>(a, L, stream);
    return launch_refresh<float>(a, L, stream);
}
