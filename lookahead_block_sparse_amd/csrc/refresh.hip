// Index refresh: Query Encoder, dual-encoder block logits, sigmoid>0.5 threshold, OR-union and
// ordered compaction of the loaded-block list (zhichai.net explainer of "FlashMemory-DeepSeek-V4",
// section 2 steps 2-3, section 3 (Query Encoder, frozen KIComp keys), section 4 (OR-mode union)).
//
// One kernel of 4-wave groups, four roles in this order of group index:
//   encode   q[r][i][j] = sum_m W_q[i][j][m] h[r][i][m]: two waves per pair of output rows, each
//            W_q row read once for every request, fp32 accumulation, q kept in fp32.
//   prefetch as many groups as fit beside the encode groups at the start: read the keys of the
//            first score units and drop them, so HBM streams keys into the memory-side cache while
//            q is computed.
//   score    one wave per unit = 32 key rows of one indexer in one 64-block word.  The wave issues
//            all loads of its rows, then waits for its q, forms z = q.k + bias in fp32, turns z > 0
//            into 32 bits with a wavefront ballot and publishes them.  Waves never synchronise with
//            the other waves of their group.
//   compact  one per 64 words of a request: waits until every unit of the request up to its words
//            has published, ORs the indexers' bits into the union words, offsets its words by the
//            popcounts before them and a wave scan, and writes their ids in ascending order; the
//            last one of a request writes the count.
// A group only waits for groups with a lower index, which were dispatched before it, and every
// wait is bounded: a wait that gives up marks the request, whose count is then written as -1.
// Values that cross groups travel in 64-bit words whose upper half is the call's number and lower
// half the value, stored and loaded with device-scope atomics: a word is valid for this call when
// its tag matches, so nothing has to be cleared between calls and no fence is needed.
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>

#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int kMaxReq = LSA_MAX_REFRESH_REQ;
constexpr int kThreads = 256;
constexpr unsigned kSpinLimit = 1u << 16;
constexpr unsigned long long kTagMask = 0xffffffff00000000ull;

struct RefreshParams {
    const void* hidden;
    long long hidden_req_stride, hidden_idx_stride;
    const void* w_q;
    const void* keys;
    const float* bias;
    int* sel_ids;
    int* sel_count;
    unsigned long long* masks;
    unsigned long long* qw;   // [n_req][n_idx][d_idx]          tag | fp32 bits of q
    unsigned long long* hw;   // [total words][n_idx][2]        tag | 32 bits of one unit
    unsigned long long* bad;  // [n_req]                        tag when a wait of the request gave up
    unsigned long long tag;   // call number << 32
    int n_req, d_model, d_idx, n_idx, n_units, n_encode_groups, n_prefetch_groups, n_score_groups;
    long long blk_off[kMaxReq + 1];
    int word_off[kMaxReq + 1];
    int cg_off[kMaxReq + 1];  // first compaction group of each request
    int2* table_out;          // optional: (id, tslot[r] + id) pairs at pair blk_off[r]
    int tslot[kMaxReq];
};

__device__ __forceinline__ void put(unsigned long long* w, unsigned long long tag, unsigned v) {
    __hip_atomic_store(w, tag | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long get(const unsigned long long* w) {
    return __hip_atomic_load(const_cast<unsigned long long*>(w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tagged(unsigned long long w, unsigned long long tag) { return (w & kTagMask) == tag; }

// The score waves read every key once per call: non-temporal 16-byte loads (about 4% faster than
// ordinary loads for the whole refresh; the prefetch role keeps ordinary loads, whose lines must stay
// in the memory-side cache for the score waves).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt(const uint4* q) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(q));
    return make_uint4(v.x, v.y, v.z, v.w);
}

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
// Query Encoder role.  A group works on rows of one indexer: group g = i*gpi + k owns the
// kEncRows*waves/2 rows from k*kEncRows*waves/2 on; waves 2m and 2m+1 sum the two halves of rows
// m*kEncRows ..: each wave loads the halves of kEncRows W_q rows and the matching halves of four
// requests' hidden states in one round (a hidden-state chunk serves every row of the wave).  Lane
// l reads 16-byte chunks l, l+64, ... of its half.
constexpr int kEncRows = 2;  // W_q rows per wave
constexpr int kEncReq = 4;   // requests per round

template <typename T>
__device__ void encode_role(const RefreshParams& p, int g) {
    using C = Chunk<T>;
    __shared__ float s_part[8][kEncRows][kEncReq];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int quads = (int)(blockDim.x >> 7);
    const int gpi = (p.d_idx + kEncRows * quads - 1) / (kEncRows * quads);
    const int i = g / gpi;
    const int j0 = ((g % gpi) * quads + (wave >> 1)) * kEncRows;
    const int half = wave & 1;
    const int hc = p.d_model / C::N / 2;  // 16-byte chunks per half row
    const T* wbase = static_cast<const T*>(p.w_q) + (size_t)i * p.d_idx * p.d_model;
    const T* hid = static_cast<const T*>(p.hidden) + (size_t)i * p.hidden_idx_stride;
    for (int r0 = 0; r0 < p.n_req; r0 += kEncReq) {
        float acc[kEncRows][kEncReq] = {};
        for (int c0 = 0; c0 < hc; c0 += 64 * 4) {
            // unconditional loads from clamped indices (masked after loading) keep all in flight
            uint4 wc[kEncRows][4];
            uint4 hv[kEncReq][4];
#pragma unroll
            for (int jj = 0; jj < kEncRows; ++jj) {
                const uint4* w = reinterpret_cast<const uint4*>(wbase + (size_t)min(j0 + jj, p.d_idx - 1) * p.d_model) + half * hc;
#pragma unroll
                for (int k = 0; k < 4; ++k) wc[jj][k] = w[min(c0 + k * 64 + lane, hc - 1)];
            }
#pragma unroll
            for (int rr = 0; rr < kEncReq; ++rr) {
                const uint4* h = reinterpret_cast<const uint4*>(hid + (size_t)min(r0 + rr, p.n_req - 1) * p.hidden_req_stride) + half * hc;
#pragma unroll
                for (int k = 0; k < 4; ++k) hv[rr][k] = h[min(c0 + k * 64 + lane, hc - 1)];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool live = c0 + k * 64 + lane < hc;
#pragma unroll
                for (int jj = 0; jj < kEncRows; ++jj)
#pragma unroll
                    for (int rr = 0; rr < kEncReq; ++rr) {
                        const float d = dot_chunks<T>(wc[jj][k], hv[rr][k]);
                        acc[jj][rr] += live ? d : 0.f;
                    }
            }
        }
#pragma unroll
        for (int jj = 0; jj < kEncRows; ++jj)
#pragma unroll
            for (int rr = 0; rr < kEncReq; ++rr) {
                const float v = wave_sum(acc[jj][rr]);
                if (lane == 0) s_part[wave][jj][rr] = v;
            }
        __syncthreads();
        if (half == 0 && lane < kEncRows * kEncReq) {
            const int jj = lane / kEncReq, rr = lane % kEncReq;
            const int j = j0 + jj;
            if (j < p.d_idx && r0 + rr < p.n_req) {
                const float q = s_part[wave][jj][rr] + s_part[wave + 1][jj][rr];
                put(&p.qw[((size_t)(r0 + rr) * p.n_idx + i) * p.d_idx + j], p.tag, __float_as_uint(q));
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------------
// Prefetch role: the groups dispatched with the encode groups read the keys of the first score
// units and drop them.  The reads pass through the memory-side cache, so HBM streams keys while q
// is being computed, and the score waves of those units later find them there.
template <typename T, int DIDX>
__device__ void prefetch_role(const RefreshParams& p, int gp) {
    constexpr int ROW_BYTES = DIDX * (int)sizeof(T);
    constexpr int LPR = ROW_BYTES / 128;
    const int lane = threadIdx.x & 63;
    const int unit = 4 * gp + (int)(threadIdx.x >> 6);
    if (unit >= p.n_units) return;
    const int word = unit / (2 * p.n_idx);
    const int i = (unit / 2) % p.n_idx;
    const int half = unit & 1;
    int r = 0;
    while (r + 1 < p.n_req && p.word_off[r + 1] <= word) ++r;
    const long long b_first = p.blk_off[r];
    const int n_blk = (int)(p.blk_off[r + 1] - b_first);
    const int b0 = (word - p.word_off[r]) * 64;
    const int n_valid = min(64, n_blk - b0);
    const char* rows = static_cast<const char*>(p.keys) + ((size_t)p.n_idx * b_first + (size_t)i * n_blk + b0) * ROW_BYTES;
    uint4 v[4][LPR];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int rowi = min(32 * half + g * 8 + (lane >> 3), n_valid - 1);
        const uint4* src = reinterpret_cast<const uint4*>(rows + (size_t)rowi * ROW_BYTES + (lane & 7) * 16);
#pragma unroll
        for (int k = 0; k < LPR; ++k) v[g][k] = src[k * 8];
    }
    uint4 x = v[0][0];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int k = 0; k < LPR; ++k) x ^= v[g][k];
    asm volatile("" :: "v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));  // the data arrives before the wave ends
}

// ------------------------------------------------------------------------------------------
// Scoring role: wave w of score group gs takes unit 4*gs + w = (word, indexer i, half): rows
// 32*half .. 32*half + 31 of the word's 64 blocks for indexer i.
template <typename T, int DIDX>
__device__ void score_role(const RefreshParams& p, int gs) {
    using C = Chunk<T>;
    constexpr int ROW_BYTES = DIDX * (int)sizeof(T);
    constexpr int LPR = ROW_BYTES / 128;  // 16-byte loads per lane per row (8 lanes per row)
    constexpr int QPL = LPR * C::N;       // q values held per lane
    constexpr int HALF = (LPR == 8) ? 2 : 1;
    constexpr int GH = 4 / HALF;          // groups of 8 rows per pass (32 rows per wave)
    constexpr int QW = DIDX / 64;         // q words fetched per lane
    static_assert(LPR >= 1 && LPR <= 8, "row size");
    __shared__ float s_q[kThreads / 64][DIDX];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int unit = 4 * gs + wave;
    if (unit >= p.n_units) return;
    const int word = unit / (2 * p.n_idx);
    const int i = (unit / 2) % p.n_idx;
    const int half = unit & 1;
    int r = 0;
    while (r + 1 < p.n_req && p.word_off[r + 1] <= word) ++r;
    const int lw = word - p.word_off[r];
    const long long b_first = p.blk_off[r];
    const int n_blk = (int)(p.blk_off[r + 1] - b_first);
    const int b0 = lw * 64;
    const int n_valid = min(64, n_blk - b0);

    const int x = lane & 7;      // 16-byte column inside a 128-byte slice of the row
    const int rsub = lane >> 3;  // row inside a group of 8 rows
    const char* rows = static_cast<const char*>(p.keys) + ((size_t)p.n_idx * b_first + (size_t)i * n_blk + b0) * ROW_BYTES;
    const unsigned long long* qrow = p.qw + ((size_t)r * p.n_idx + i) * DIDX;
    const float bias = p.bias[r * p.n_idx + i];
    unsigned bits = 0u;
    bool q_ok = true;
    float qr[QPL];
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
            for (int k = 0; k < LPR; ++k) v[g][k] = load_nt(src + k * 8);
        }
        if (hh == 0) {
            asm volatile("" ::: "memory");  // the key loads are issued before the wait for q
            // wait for this (request, indexer)'s q: the wave fetches the row (lane l: words QW*l ..)
            // right behind its key loads, checks every tag (fetching again until all are this
            // call's) and passes the values through LDS to the lanes that use them
            unsigned spins = 0;
            for (;;) {
                bool all = true;
#pragma unroll
                for (int k = 0; k < QW; ++k) {
                    const unsigned long long wq = get(qrow + QW * lane + k);
                    all = all && tagged(wq, p.tag);
                    s_q[wave][QW * lane + k] = __uint_as_float((unsigned)wq);
                }
                if (__all(all)) break;
                if (++spins > kSpinLimit) {
                    q_ok = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int k = 0; k < LPR; ++k)
#pragma unroll
                for (int e = 0; e < C::N; ++e) qr[k * C::N + e] = s_q[wave][(k * 128 + x * 16) / (int)sizeof(T) + e];
        }
#pragma unroll
        for (int g = 0; g < GH; ++g) {
            const int rowi = 32 * half + (hh * GH + g) * 8 + rsub;
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < LPR; ++k) acc += dot_chunk_f32<T>(v[g][k], qr + k * C::N);
            acc += __shfl_xor(acc, 1, 64);
            acc += __shfl_xor(acc, 2, 64);
            acc += __shfl_xor(acc, 4, 64);
            const bool keep = q_ok && (rowi < n_valid) && (acc + bias > 0.f);
            const unsigned long long m = __ballot(keep);
            unsigned b8 = 0u;  // lanes 8j..8j+7 all hold row 8g+j: take bit 8j
#pragma unroll
            for (int j = 0; j < 8; ++j) b8 |= (unsigned)((m >> (8 * j)) & 1ull) << j;
            bits |= b8 << (8 * (hh * GH + g));
        }
    }
    if (lane == 0) {
        if (p.masks) {
            const int n_words_r = p.word_off[r + 1] - p.word_off[r];
            const size_t mw = (size_t)(p.n_idx + 1) * p.word_off[r] + (size_t)i * n_words_r + lw;
            reinterpret_cast<unsigned*>(p.masks)[2 * mw + half] = bits;
        }
        if (!q_ok) {
            put(&p.bad[r], p.tag, 1u);
            __builtin_amdgcn_s_waitcnt(0);  // the mark is stored before the unit is published
        }
        put(&p.hw[unit], p.tag, bits);
    }
}

// ------------------------------------------------------------------------------------------
// Compaction role: group c of a request handles the request's words [64c, 64c + 64) (its slice).
// All 256 threads read the union words up to the slice's end (thread t: words t, t+256, ...) until
// every unit carries this call's tag; the popcounts of the words before the slice give its base,
// a wave scan over the slice gives each word's offset, and the four waves write the slice's ids,
// one word at a time per wave with one lane per bit, so each store writes a word's ids contiguously.
// The group of the last slice writes the count.
constexpr int kSlice = 64;

__device__ void compact_role(const RefreshParams& p, int cg) {
    __shared__ unsigned long long s_u[kSlice];
    __shared__ int s_pos[kSlice];
    __shared__ int s_sum[kThreads / 64];
    __shared__ int s_total;
    int r = 0;
    while (r + 1 < p.n_req && p.cg_off[r + 1] <= cg) ++r;
    const int c = cg - p.cg_off[r];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int n_words = p.word_off[r + 1] - p.word_off[r];
    const int s0 = c * kSlice;
    const int s1 = min(n_words, s0 + kSlice);
    const int nh = 2 * p.n_idx;  // published units per word
    const unsigned long long* hw = p.hw + (size_t)p.word_off[r] * nh;
    auto union_word = [&](int w, bool* ok) {
        // all loads of the word first (n_idx <= 4: at most 8 units), then the checks
        unsigned long long h[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) h[k] = get(hw + (size_t)w * nh + min(k, nh - 1));
        unsigned long long u = 0ull;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (k < nh) {
                *ok = *ok && tagged(h[k], p.tag);
                u |= (unsigned long long)(unsigned)h[k] << (32 * (k & 1));
            }
        }
        return u;
    };
    // Runs of up to kKeep words per thread stay in registers: a word is read until all its units
    // carry this call's tag, then kept; requests longer than 256*kKeep words are re-read.
    constexpr int kKeep = 4;
    const bool held = s1 <= kThreads * kKeep;
    unsigned long long keep[kKeep] = {};
    unsigned done = 0u;
    bool failed = false;
    bool bad = false;
    for (unsigned spins = 0;; ++spins) {
        bool ok = true;
        if (held) {
#pragma unroll
            for (int k = 0; k < kKeep; ++k) {
                const int w = t + kThreads * k;
                if (w < s1 && !((done >> k) & 1u)) {
                    bool okw = true;
                    const unsigned long long u = union_word(w, &okw);
                    if (okw) {
                        keep[k] = u;
                        done |= 1u << k;
                    } else {
                        ok = false;
                    }
                }
            }
        } else {
            for (int w = t; w < s1; w += kThreads) union_word(w, &ok);
        }
        if (t == 0) bad = tagged(get(&p.bad[r]), p.tag);
        if (__syncthreads_and(ok)) break;
        if (spins >= kSpinLimit) {
            failed = true;
            if (t == 0) put(&p.bad[r], p.tag, 1u);
            break;
        }
        __builtin_amdgcn_s_sleep(4);
    }
    // popcounts before the slice; the slice's words to LDS
    int before = 0;
    if (held) {
#pragma unroll
        for (int k = 0; k < kKeep; ++k) {
            const int w = t + kThreads * k;
            if (w < s0)
                before += __popcll(keep[k]);
            else if (w < s1)
                s_u[w - s0] = keep[k];
        }
    } else {
        for (int w = t; w < s1; w += kThreads) {
            bool ok = true;
            const unsigned long long u = union_word(w, &ok);
            if (w < s0)
                before += __popcll(u);
            else
                s_u[w - s0] = u;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) before += __shfl_xor(before, o, 64);
    if (lane == 0) s_sum[wave] = before;
    __syncthreads();
    if (wave == 0) {
        int base = 0;
#pragma unroll
        for (int k = 0; k < kThreads / 64; ++k) base += s_sum[k];
        const unsigned long long u = lane < s1 - s0 ? s_u[lane] : 0ull;
        const int cnt = __popcll(u);
        int inc = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(inc, o, 64);
            if (lane >= o) inc += v;
        }
        s_pos[lane] = base + inc - cnt;
        if (lane == 63) s_total = base + inc;
    }
    __syncthreads();
    if (!failed) {
        int* out = p.sel_ids + p.blk_off[r];
        const size_t plane = (size_t)(p.n_idx + 1) * p.word_off[r] + (size_t)p.n_idx * n_words;
        if (p.masks && t < s1 - s0) p.masks[plane + s0 + t] = s_u[t];
        // wave w writes slice words w, w+4, ..: lane m first fetches word w + 4m, then the words go
        // to scalars one at a time
        constexpr int kPerWave = kSlice / (kThreads / 64);
        const int jm = wave + (kThreads / 64) * (lane % kPerWave);
        const unsigned long long um = jm < s1 - s0 ? s_u[jm] : 0ull;
        const int pm = s_pos[jm < kSlice ? jm : 0];
        const int ulo = (int)(unsigned)um, uhi = (int)(unsigned)(um >> 32);
#pragma unroll
        for (int m = 0; m < kPerWave; ++m) {
            const unsigned long long u = (unsigned long long)(unsigned)__builtin_amdgcn_readlane(ulo, m) |
                                         ((unsigned long long)(unsigned)__builtin_amdgcn_readlane(uhi, m) << 32);
            const int at = __builtin_amdgcn_readlane(pm, m);
            const int j = wave + (kThreads / 64) * m;
            if ((u >> lane) & 1ull) {
                const int pos = at + __popcll(u & ((1ull << lane) - 1ull));
                const int id = (s0 + j) * 64 + lane;
                out[pos] = id;
                if (p.table_out) p.table_out[p.blk_off[r] + pos] = make_int2(id, p.tslot[r] + id);
            }
        }
    }
    if (t == 0 && s1 == n_words) p.sel_count[r] = (failed || bad) ? -1 : s_total;
}

template <typename T, int DIDX>
__global__ __launch_bounds__(kThreads, 3) void refresh_kernel(RefreshParams p) {
    int g = blockIdx.x;
    if (g < p.n_encode_groups) {
        encode_role<T>(p, g);
        return;
    }
    g -= p.n_encode_groups;
    if (g < p.n_prefetch_groups) {
        prefetch_role<T, DIDX>(p, g);
        return;
    }
    g -= p.n_prefetch_groups;
    if (g < p.n_score_groups)
        score_role<T, DIDX>(p, g);
    else
        compact_role(p, g - p.n_score_groups);
}

struct RefreshLayout {
    size_t qw_off, hw_off, bad_off, total;
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
    LSA_CHECK_ARG(words <= (1ll << 26), "lsa_index_refresh: too many blocks");
    L->total_words = (int)words;
    size_t off = 0;
    L->qw_off = off;
    off = align_up(off + (size_t)a->n_req * a->n_idx * a->d_idx * sizeof(unsigned long long), 256);
    L->hw_off = off;
    off = align_up(off + (size_t)words * 2 * a->n_idx * sizeof(unsigned long long), 256);
    L->bad_off = off;
    off = align_up(off + (size_t)a->n_req * sizeof(unsigned long long), 256);
    L->total = off;
    return LSA_OK;
}

// Call numbers tag the workspace words of a call; 0 never occurs, so a zero-filled workspace holds
// no valid word.
std::atomic<unsigned> g_call_number{0};

template <typename T>
lsa_status launch_refresh(const lsa_refresh_args* a, const RefreshLayout& L, hipStream_t stream) {
    char* ws = static_cast<char*>(a->workspace);
    unsigned call = g_call_number.fetch_add(1u) + 1u;
    if (call == 0u) call = g_call_number.fetch_add(1u) + 1u;
    RefreshParams rp{};
    rp.hidden = a->hidden;
    rp.hidden_req_stride = a->hidden_req_stride;
    rp.hidden_idx_stride = a->hidden_idx_stride;
    rp.w_q = a->w_q;
    rp.keys = a->keys;
    rp.bias = a->bias;
    rp.sel_ids = a->sel_ids;
    rp.sel_count = a->sel_count;
    rp.masks = reinterpret_cast<unsigned long long*>(a->masks);
    rp.table_out = reinterpret_cast<int2*>(a->table_out);
    for (int r = 0; r < a->n_req; ++r) rp.tslot[r] = a->table_out ? a->table_slot_base[r] : 0;
    rp.qw = reinterpret_cast<unsigned long long*>(ws + L.qw_off);
    rp.hw = reinterpret_cast<unsigned long long*>(ws + L.hw_off);
    rp.bad = reinterpret_cast<unsigned long long*>(ws + L.bad_off);
    rp.tag = (unsigned long long)call << 32;
    rp.n_req = a->n_req;
    rp.d_model = a->d_model;
    rp.d_idx = a->d_idx;
    rp.n_idx = a->n_idx;
    rp.n_units = L.total_words * 2 * a->n_idx;
    const int rows_per_group = kEncRows * (kThreads / 128);  // two waves per kEncRows W_q rows
    rp.n_encode_groups = a->n_idx * ((a->d_idx + rows_per_group - 1) / rows_per_group);
    rp.n_score_groups = (rp.n_units + kThreads / 64 - 1) / (kThreads / 64);
    int wo = 0, co = 0;
    for (int r = 0; r <= a->n_req; ++r) {
        rp.blk_off[r] = a->blk_off[r];
        rp.word_off[r] = wo;
        rp.cg_off[r] = co;
        if (r < a->n_req) {
            const int nw = (int)((a->blk_off[r + 1] - a->blk_off[r] + 63) / 64);
            wo += nw;
            co += (nw + kSlice - 1) / kSlice;
        }
    }
    auto kernel = a->d_idx == 256 ? refresh_kernel<T, 256> : refresh_kernel<T, 128>;
    // prefetch groups fill the slots the encode groups leave free at the start
    {
        DeviceInfo dev;
        lsa_status st = current_device(&dev);
        if (st != LSA_OK) return st;
        int per_cu = 0;
        LSA_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0));
        rp.n_prefetch_groups = std::max(0, std::min(rp.n_score_groups, dev.cu_count * per_cu - rp.n_encode_groups));
    }
    const dim3 grid(rp.n_encode_groups + rp.n_prefetch_groups + rp.n_score_groups + co), block(kThreads);
    if (a->ev_begin && a->ev_end)  // the events take the dispatch's own start and end timestamps
        hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, a->ev_begin, a->ev_end, 0, rp);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, rp);
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
    if (a->table_out) {
        LSA_CHECK_ARG(a->table_slot_base != nullptr, "lsa_index_refresh: table_out without table_slot_base");
        LSA_CHECK_ARG(((uintptr_t)a->table_out % 8) == 0, "lsa_index_refresh: table_out must be 8-byte aligned");
        for (int r = 0; r < a->n_req; ++r) {
            const long long base = a->table_slot_base[r], nb = a->blk_off[r + 1] - a->blk_off[r];
            LSA_CHECK_ARG(base >= 0 && base + nb <= 0x7fffffffll,
                          "lsa_index_refresh: table_slot_base[%d]=%lld puts slots outside int32", r, base);
        }
    }
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
