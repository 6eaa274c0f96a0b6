// Index refresh: Query Encoder, dual-encoder block logits, sigmoid>0.5 threshold, OR-union and
// ordered compaction of the loaded-block list (zhichai.net explainer of "FlashMemory-DeepSeek-V4",
// section 2 steps 2-3, section 3 (Query Encoder, frozen KIComp keys), section 4 (OR-mode union)).
//
// One launch of 4-wave groups, three roles in this order of group index:
//   encode   q[r][i][j] = sum_m W_q[i][j][m] h[r][i][m]: a wave owns two whole output rows of one
//            indexer for four requests; it requests both W_q rows and the four hidden states in
//            one batch, accumulates in fp32 and publishes the eight values of q (kept in fp32).
//   score    one wave per half of a 64-block word (32 blocks), all indexers: for each indexer the
//            32 key rows are contiguous and read as whole 1 KiB runs (lane l takes bytes 16 l ..
//            16 l + 15 of each run, so a lane works on one fixed 16-byte column of its rows and
//            needs only the matching 4 or 8 values of q).  The wave requests the rows of up to
//            three indexers (48 KiB) at once, then waits for q, forms z = q.k + bias in fp32 (per-
//            lane partial dot products, then a reduce-scatter across the lanes of a row), turns
//            z > 0 into 32 bits per indexer with a wavefront ballot, ORs the indexers and publishes
//            the 32 union bits of its half word.
//   compact  one per 64 words of a request: waits until every half word of the request up to its
//            words has published, offsets its words by the popcounts before them and a wave scan,
//            and writes their ids in ascending order; the last one of a request writes the count.
//   Without ids (sel_ids NULL: a caller that ranks the selected blocks from the union plane itself)
//   the score waves write their 32 union bits straight into the union plane, no compaction group is
//   launched, and the launch ends with the last score wave (~3 us earlier at 4 x 1M).
// Why the score waves hold so much: a value handed from one compute unit to another inside a
// launch (q here) travels through the memory-side queues and, with the key stream in flight,
// reaches the score waves ~10 us after the launch starts whatever the rest of the design does.
// Two groups of 48 KiB waves per compute unit request about 80% of all key bytes at the start of
// the launch, and a wave asks for q right behind its keys for all its indexers at once, so the
// memory system streams at full rate while q is computed and the wait for q is hidden behind the
// keys.  Measured alternatives at 4 x 1M context: one wave per 16 KiB unit at five groups per
// compute unit (q arrives late and holds the slots: 29-33 us), two launches (encode, then score:
// q is simply there, but the memory idles during the encode launch and the gap, 4.5 + 2.1 us:
// 30 us), fewer resident groups to keep the queues short (31-35 us), score waves that wait up to
// 2 us before their key loads so that W_q is served first (no gain), and the half words beyond
// the first round staged in LDS by direct-to-LDS loads, so that every key byte is requested at
// the start (the stream then ran at ~4.3 TB/s and the staged words were scored after a group
// barrier: 33-36 us).  The cross-lane moves of the scoring are row swaps and DPP (no LDS
// crossbar), and bf16 keys are dotted with q on v_dot2_f32_bf16, q taken as two bf16 parts (its
// value rounded to nearest even plus the rounded remainder, ~2^-18 relative); the launch is bound
// by the key stream and the hand-offs, and without compaction groups the last waves' scoring is
// its tail (the cheaper dot products and a one-round-trip q poll took ~0.6 us off it).
// A group only waits for groups with a lower index, which were dispatched before it, and every
// wait is bounded: a wait that gives up marks the request, whose count is then written as -1.
// Values that cross groups travel in 64-bit words whose upper half is the call's number and lower
// half the value, stored and loaded with device-scope atomics: a word is valid for this call when
// its tag matches, so nothing has to be cleared between calls and no fence is needed.
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <cmath>

#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int kMaxReq = LSA_MAX_REFRESH_REQ;
constexpr int kThreads = 256;
constexpr int kGroupsPerCU = 2;
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
    unsigned long long* hw;   // [total words][2]               tag | union bits of one half word
    unsigned long long* bad;  // [n_req]                        tag when a wait of the request gave up
    unsigned long long tag;   // call number << 32
    float select_logit;       // a block is kept when z > this (logit of the selection level)
    int n_req, d_model, d_idx, n_idx, n_halves, n_encode_waves, n_encode_groups, n_score_groups;
    long long blk_off[kMaxReq + 1];
    int word_off[kMaxReq + 1];
    int cg_off[kMaxReq + 1];  // first compaction group of each request
    int2* table_out;          // optional: (id, tslot[r] + id) pairs at pair blk_off[r]
    float* logits;            // optional: z at element n_idx * blk_off[r] + i * B_r + b
    int bits_only;            // no ids: the score waves write the union plane, no compaction groups
    int tslot[kMaxReq];
};

__device__ __forceinline__ void put(unsigned long long* w, unsigned long long tag, unsigned v) {
    __hip_atomic_store(w, tag | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long get(const unsigned long long* w) {
    return __hip_atomic_load(const_cast<unsigned long long*>(w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool tagged(unsigned long long w, unsigned long long tag) { return (w & kTagMask) == tag; }

// Keys and W_q are read once per call: non-temporal 16-byte loads.
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

// acc + sum of the 8 (bf16) or 4 (fp32) products of two 16-byte chunks, in fp32.  bf16 uses the
// packed two-pair dot product (v_dot2_f32_bf16: products of bf16 values are exact in fp32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ float dot_chunks(uint4 a, uint4 b, float acc);

template <>
__device__ __forceinline__ float dot_chunks<uint16_t>(uint4 a, uint4 b, float acc) {
    auto bf2 = [](unsigned w) { return __builtin_bit_cast(bf16x2, w); };
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf2(a.x), bf2(b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf2(a.y), bf2(b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf2(a.z), bf2(b.z), acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(bf2(a.w), bf2(b.w), acc, false);
}

template <>
__device__ __forceinline__ float dot_chunks<float>(uint4 a, uint4 b, float acc) {
    acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
    acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
    acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
    return fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
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
// Query Encoder role.  Encode wave e = ((i*gpi + k)*n_quads + m) owns rows 2k and 2k+1 of indexer
// i (gpi = d_idx/2 row pairs per indexer) for requests 4m .. 4m+3.  A row is read in chunks of
// kEncPieces 16-byte pieces per lane (the whole row when d_model <= 4096 for bf16, 2048 for fp32);
// per chunk the wave loads both W_q rows and the four hidden states before any is used.
constexpr int kEncReq = 4;     // requests per encode wave
constexpr int kEncRows = 2;    // W_q rows per encode wave
constexpr int kEncPieces = 8;  // 16-byte pieces per lane per row and chunk

// pieces c0 + lane + 64 k (k < kEncPieces) of a row of hc pieces, every load at a fixed distance
// from the lane's first; in the last chunk of a short row the indices are clamped to the row's
// last piece (the caller drops those pieces when it uses them, so no load waits for another)
template <bool NT>
__device__ __forceinline__ void enc_chunk(uint4* v, const uint4* row, int c0, int hc, int lane) {
    if (c0 + 64 * kEncPieces <= hc) {
#pragma unroll
        for (int k = 0; k < kEncPieces; ++k)
            v[k] = NT ? load_nt(row + c0 + lane + k * 64) : row[c0 + lane + k * 64];
    } else {
#pragma unroll
        for (int k = 0; k < kEncPieces; ++k) {
            const int idx = min(c0 + k * 64 + lane, hc - 1);
            v[k] = NT ? load_nt(row + idx) : row[idx];
        }
    }
}

template <typename T>
__device__ void encode_role(const RefreshParams& p, int e) {
    using C = Chunk<T>;
    const int lane = threadIdx.x & 63;
    const int n_quads = (p.n_req + kEncReq - 1) / kEncReq;
    const int gpi = (p.d_idx + kEncRows - 1) / kEncRows;
    const int r0 = (e % n_quads) * kEncReq;
    const int i = e / n_quads / gpi;
    const int j0 = (e / n_quads % gpi) * kEncRows;
    const int hc = p.d_model / C::N;  // 16-byte pieces per row (a multiple of 32)
    const T* wbase = static_cast<const T*>(p.w_q) + (size_t)i * p.d_idx * p.d_model;
    const T* hid = static_cast<const T*>(p.hidden) + (size_t)i * p.hidden_idx_stride;
    float acc[kEncRows][kEncReq] = {};
    for (int c0 = 0; c0 < hc; c0 += 64 * kEncPieces) {
        uint4 wv[kEncRows][kEncPieces];
        uint4 hv[kEncReq][kEncPieces];
#pragma unroll
        for (int jj = 0; jj < kEncRows; ++jj)
            enc_chunk<true>(wv[jj], reinterpret_cast<const uint4*>(wbase + (size_t)min(j0 + jj, p.d_idx - 1) * p.d_model),
                            c0, hc, lane);
#pragma unroll
        for (int rr = 0; rr < kEncReq; ++rr)
            enc_chunk<false>(hv[rr], reinterpret_cast<const uint4*>(hid + (size_t)min(r0 + rr, p.n_req - 1) *
                                                                          p.hidden_req_stride),
                             c0, hc, lane);
        __builtin_amdgcn_sched_barrier(0);  // every load of the chunk is issued before the first use
#pragma unroll
        for (int k = 0; k < kEncPieces; ++k) {
            if (c0 + k * 64 + lane >= hc) {  // a clamped piece past the row's end adds nothing
#pragma unroll
                for (int jj = 0; jj < kEncRows; ++jj) wv[jj][k] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                for (int rr = 0; rr < kEncReq; ++rr) hv[rr][k] = make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int jj = 0; jj < kEncRows; ++jj)
#pragma unroll
                for (int rr = 0; rr < kEncReq; ++rr) acc[jj][rr] = dot_chunks<T>(wv[jj][k], hv[rr][k], acc[jj][rr]);
        }
    }
    float mine = 0.f;  // lane jj*kEncReq + rr publishes q for row j0 + jj, request r0 + rr
#pragma unroll
    for (int jj = 0; jj < kEncRows; ++jj)
#pragma unroll
        for (int rr = 0; rr < kEncReq; ++rr) {
            const float v = wave_sum(acc[jj][rr]);
            if (lane == jj * kEncReq + rr) mine = v;
        }
    const int jj = lane / kEncReq, rr = lane % kEncReq;
    if (lane < kEncRows * kEncReq && j0 + jj < p.d_idx && r0 + rr < p.n_req)
        put(&p.qw[((size_t)(r0 + rr) * p.n_idx + i) * p.d_idx + j0 + jj], p.tag, __float_as_uint(mine));
}

// ------------------------------------------------------------------------------------------
// Scoring role.  Score wave s takes half word s: word s/2, blocks 32*(s%2) .. +31, for every
// indexer.  For indexer i the half word's 32 key rows (ROW bytes each) are contiguous; load j of
// the unit reads 1 KiB run j: lane l holds 16-byte column c = l % LPR of row RPL*j + l / LPR.
// After the loads each lane has one partial dot product per run (its column); a reduce-scatter
// halves the partials at each step over the top lane bits of a row's lanes and sums the rest,
// leaving lane l with the logit of run k = (l >> (LOG_LPR - LOG_P)) % P, i.e. of row
// RPL*k + l / LPR.  Up to U units (indexers) are requested at once.
template <typename T, int DIDX>
struct ScoreShape {
    static constexpr int ROW = DIDX * (int)sizeof(T);  // bytes per key row: 256, 512 or 1024
    static constexpr int LPR = ROW / 16;               // lanes per row
    static constexpr int LOG_LPR = LPR == 16 ? 4 : LPR == 32 ? 5 : 6;
    static constexpr int RPL = 64 / LPR;               // rows per 1 KiB run
    static constexpr int P = 32 * ROW / 1024;          // runs per unit: 8, 16 or 32
    static constexpr int LOG_P = P == 8 ? 3 : P == 16 ? 4 : 5;
    static constexpr int U = 48 / P;                   // units requested at once: 6, 3 or 1
    static constexpr int E = Chunk<T>::N;              // elements of q per lane (its column)
    static constexpr int QF = E / RPL;                 // of which the lane fetches (RPL lanes share a column)
    static_assert(P * RPL == 32, "a unit is 32 rows");
    static_assert(QF * RPL == E, "q split over the lanes of a column");
    static_assert(LOG_P <= LOG_LPR, "reduce-scatter shape");
};

// Cross-lane moves for the score role, all full-rate (no LDS crossbar): the 16-lane row swap and
// the half-wave swap exchange whole rows / halves; row mirror (lane ^ 15), half-row mirror
// (lane ^ 7) and the quad permutations pair lanes whose index differs in bit 3, 2, 1 or 0 and
// agrees in the bits above it.
__device__ __forceinline__ float as_f(unsigned x) { return __uint_as_float(x); }
__device__ __forceinline__ unsigned as_u(float x) { return __float_as_uint(x); }
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
template <int B>
__device__ __forceinline__ float dpp_partner(float x) {  // the value of a lane differing in bit B
    static_assert(B >= 0 && B <= 3, "row-local pairing");
    if constexpr (B == 3) return dpp<0x140>(x);  // row_mirror
    else if constexpr (B == 2) return dpp<0x141>(x);  // row_half_mirror
    else if constexpr (B == 1) return dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    else return dpp<0xB1>(x);                          // quad_perm [1, 0, 3, 2]
}
// One reduce-scatter step over lane bit B on the n entries of v: a lane with bit B set keeps the
// upper half, the others the lower half, each adding its partner's copy of the half it keeps.
template <int B, int N>
__device__ __forceinline__ void rs_step(float* v, int lane) {
    if constexpr (B >= 4) {
#pragma unroll
        for (int kk = 0; kk < N / 2; ++kk) {
            // the swap leaves each lane its own copy and its partner's copy of the half it keeps
            const auto x = B == 4 ? __builtin_amdgcn_permlane16_swap(as_u(v[kk]), as_u(v[kk + N / 2]), false, false)
                                  : __builtin_amdgcn_permlane32_swap(as_u(v[kk]), as_u(v[kk + N / 2]), false, false);
            v[kk] = as_f(x[0]) + as_f(x[1]);
        }
    } else {
        const bool up = (lane >> B) & 1;
#pragma unroll
        for (int kk = 0; kk < N / 2; ++kk) {
            const float keep = up ? v[kk + N / 2] : v[kk];
            const float give = up ? v[kk] : v[kk + N / 2];
            v[kk] = keep + dpp_partner<B>(give);
        }
    }
}
template <int B, int N, int STEPS>
__device__ __forceinline__ void rs_steps(float* v, int lane) {
    if constexpr (STEPS > 0) {
        rs_step<B, N>(v, lane);
        rs_steps<B - 1, N / 2, STEPS - 1>(v, lane);
    }
}
// the value of lane (l mod LPR) + s LPR for s < 64 / LPR (rows of a 1 KiB run), for every lane l
template <int RPL>
__device__ __forceinline__ void gather_rows(float x, float* out) {
    if constexpr (RPL == 1) {
        out[0] = x;
    } else if constexpr (RPL == 2) {
        const auto h = __builtin_amdgcn_permlane32_swap(as_u(x), as_u(x), false, false);
        out[0] = as_f(h[0]);  // lower half's value
        out[1] = as_f(h[1]);  // upper half's value
    } else {
        static_assert(RPL == 4, "rows per run");
        const auto h = __builtin_amdgcn_permlane32_swap(as_u(x), as_u(x), false, false);
        const auto a = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);  // rows 0, 1
        const auto b = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);  // rows 2, 3
        out[0] = as_f(a[0]);
        out[1] = as_f(a[1]);
        out[2] = as_f(b[0]);
        out[3] = as_f(b[1]);
    }
}

// fp32 -> bf16 bits, rounded to nearest even (finite values)
__device__ __forceinline__ unsigned bf16_rne(float x) {
    const unsigned u = __float_as_uint(x);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Where half word sw lives: its request, word and row base.
struct HalfWord {
    int sw, half, r, lw, n_blk, n_valid;
    const char* word_rows;  // indexer i's rows of the word start at word_rows + i * n_blk * ROW
};
template <int ROW>
__device__ __forceinline__ HalfWord half_word(const RefreshParams& p, int sw) {
    HalfWord h;
    h.sw = sw;
    const int word = sw >> 1;
    h.half = sw & 1;
    int r = 0;
    while (r + 1 < p.n_req && p.word_off[r + 1] <= word) ++r;
    h.r = r;
    h.lw = word - p.word_off[r];
    const long long b_first = p.blk_off[r];
    h.n_blk = (int)(p.blk_off[r + 1] - b_first);
    h.n_valid = min(64, h.n_blk - h.lw * 64);  // blocks of this word that exist (>= 1)
    h.word_rows = static_cast<const char*>(p.keys) + ((size_t)p.n_idx * b_first + h.lw * 64) * ROW;
    return h;
}

// The key runs of indexers i0 .. i0 + nu - 1 of a half word into registers: run j of unit u at a
// fixed distance from the unit's first row; in the request's last word a lane whose row lies past
// the request's last block loads nothing (its logit is masked), so every access stays inside the
// request's keys.
template <typename T, int DIDX>
__device__ __forceinline__ void load_runs(const HalfWord& h, int i0, int nu, int lane, uint4 (&v)[ScoreShape<T, DIDX>::U][ScoreShape<T, DIDX>::P]) {
    using S = ScoreShape<T, DIDX>;
    const int sub = lane / S::LPR;
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
        if (u < nu) {
            const char* rows = h.word_rows + ((size_t)(i0 + u) * h.n_blk + 32 * h.half) * S::ROW + lane * 16;
            if (h.n_valid == 64) {
#pragma unroll
                for (int j = 0; j < S::P; ++j) v[u][j] = load_nt(reinterpret_cast<const uint4*>(rows + j * 1024));
            } else {
#pragma unroll
                for (int j = 0; j < S::P; ++j) {
                    v[u][j] = make_uint4(0u, 0u, 0u, 0u);
                    if (32 * h.half + S::RPL * j + sub < h.n_valid)
                        v[u][j] = load_nt(reinterpret_cast<const uint4*>(rows + j * 1024));
                }
            }
        }
    }
}

// Logits of a half word's rows for indexers i0 .. i0 + nu - 1 (keys in v), thresholded and ORed
// into u_bits.  q of every indexer of the batch is polled together: lane l fetches QF of the E
// values of its column (the RPL lanes of a column split them) and fetches again until every tag is
// this call's.
template <typename T, int DIDX>
__device__ __forceinline__ void score_runs(const RefreshParams& p, const HalfWord& h, int i0, int nu, int lane,
                                           const uint4 (&v)[ScoreShape<T, DIDX>::U][ScoreShape<T, DIDX>::P],
                                           unsigned* u_bits, bool* q_ok) {
    using S = ScoreShape<T, DIDX>;
    const int col = lane % S::LPR;
    const int sub = lane / S::LPR;
    const int k = (lane >> (S::LOG_LPR - S::LOG_P)) & (S::P - 1);
    const int rowi = 32 * h.half + S::RPL * k + sub;  // row of the word whose logit this lane ends with
    float qf[S::U][S::QF];
    for (unsigned spins = 0;; ++spins) {
        // every load unconditional (units past nu read the last indexer's row, and are ignored), so
        // that the whole poll is one round trip rather than one per unit
        unsigned long long wq[S::U][S::QF];
#pragma unroll
        for (int u = 0; u < S::U; ++u) {
            const int iu = min(i0 + u, p.n_idx - 1);
            const unsigned long long* qrow = p.qw + ((size_t)h.r * p.n_idx + iu) * DIDX + col * S::E + sub * S::QF;
#pragma unroll
            for (int e = 0; e < S::QF; ++e) wq[u][e] = get(qrow + e);
        }
        bool all = true;
#pragma unroll
        for (int u = 0; u < S::U; ++u)
#pragma unroll
            for (int e = 0; e < S::QF; ++e) {
                all &= u >= nu || tagged(wq[u][e], p.tag);
                qf[u][e] = __uint_as_float((unsigned)wq[u][e]);
            }
        if (__all(all)) break;
        if (spins >= kSpinLimit) {
            *q_ok = false;
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int u = 0; u < S::U; ++u) {
        if (u < nu) {
            const int i = i0 + u;
            float part[S::P];
            if constexpr (sizeof(T) == 2) {
                // bf16 keys: q as two bf16 parts, hi = q rounded to nearest even and lo = (q - hi)
                // rounded likewise (hi + lo is q to ~2^-17 relative, far inside the logit margin),
                // packed in pairs by the lane that fetched them, gathered, and dotted with the keys
                // on v_dot2_f32_bf16 (products of bf16 values are exact in fp32)
                constexpr int QP = S::QF / 2;  // packed pairs this lane fetched
                unsigned ph[QP], pl[QP];
#pragma unroll
                for (int e2 = 0; e2 < QP; ++e2) {
                    const float a = qf[u][2 * e2], b = qf[u][2 * e2 + 1];
                    const unsigned ha = bf16_rne(a), hb = bf16_rne(b);
                    const unsigned la = bf16_rne(a - __uint_as_float(ha << 16)), lb = bf16_rne(b - __uint_as_float(hb << 16));
                    ph[e2] = ha | (hb << 16);
                    pl[e2] = la | (lb << 16);
                }
                unsigned qh[S::E / 2], ql[S::E / 2];  // the column's E values as pairs, lane order
#pragma unroll
                for (int e2 = 0; e2 < QP; ++e2) {
                    float gh[S::RPL], gl[S::RPL];
                    gather_rows<S::RPL>(__uint_as_float(ph[e2]), gh);
                    gather_rows<S::RPL>(__uint_as_float(pl[e2]), gl);
#pragma unroll
                    for (int s2 = 0; s2 < S::RPL; ++s2) {
                        qh[s2 * QP + e2] = __float_as_uint(gh[s2]);
                        ql[s2 * QP + e2] = __float_as_uint(gl[s2]);
                    }
                }
                const uint4 qh4 = make_uint4(qh[0], qh[1], qh[2], qh[3]);
                const uint4 ql4 = make_uint4(ql[0], ql[1], ql[2], ql[3]);
#pragma unroll
                for (int j = 0; j < S::P; ++j) part[j] = dot_chunks<T>(v[u][j], ql4, dot_chunks<T>(v[u][j], qh4, 0.f));
            } else {
                float qv[S::E];  // the column's E values, gathered from the lanes that fetched them
#pragma unroll
                for (int e = 0; e < S::QF; ++e) {
                    float g[S::RPL];
                    gather_rows<S::RPL>(qf[u][e], g);
#pragma unroll
                    for (int s2 = 0; s2 < S::RPL; ++s2) qv[s2 * S::QF + e] = g[s2];
                }
#pragma unroll
                for (int j = 0; j < S::P; ++j) part[j] = dot_chunk_f32<T>(v[u][j], qv);
            }
            // reduce-scatter: step t keeps the upper half of the remaining partials on lanes
            // whose bit (LOG_LPR - 1 - t) is set and adds the partner lane's copy of that half
            rs_steps<S::LOG_LPR - 1, S::P, S::LOG_P>(part, lane);
            float z = part[0];
            if constexpr (S::LOG_LPR - S::LOG_P == 2) z += dpp_partner<1>(z);
            if constexpr (S::LOG_LPR - S::LOG_P >= 1) z += dpp_partner<0>(z);
            static_assert(S::LOG_LPR - S::LOG_P <= 2, "row lanes left after the reduce-scatter");
            const float zb = z + p.bias[h.r * p.n_idx + i];
            const bool keep = *q_ok && (rowi < h.n_valid) && (zb > p.select_logit);
            // the lanes that share a row hold the same logit: the first of them stores it
            if (p.logits && rowi < h.n_valid && (lane & ((1 << (S::LOG_LPR - S::LOG_P)) - 1)) == 0)
                p.logits[(size_t)p.n_idx * p.blk_off[h.r] + (size_t)i * h.n_blk + h.lw * 64 + rowi] = zb;
            const unsigned long long m = __ballot(keep);
            // row q of the half word sits on lane (q % RPL) * LPR + ((q / RPL) << (LOG_LPR - LOG_P))
            unsigned bits = 0u;
#pragma unroll
            for (int q = 0; q < 32; ++q) {
                const int ln = (q % S::RPL) * S::LPR + ((q / S::RPL) << (S::LOG_LPR - S::LOG_P));
                bits |= (unsigned)((m >> ln) & 1ull) << q;
            }
            *u_bits |= bits;
            if (p.masks && lane == 0) {
                const int n_words_r = p.word_off[h.r + 1] - p.word_off[h.r];
                const size_t mw = (size_t)(p.n_idx + 1) * p.word_off[h.r] + (size_t)i * n_words_r + h.lw;
                reinterpret_cast<unsigned*>(p.masks)[2 * mw + h.half] = bits;
            }
        }
    }
}

__device__ __forceinline__ void publish_half(const RefreshParams& p, const HalfWord& h, unsigned u_bits, bool q_ok,
                                             int lane) {
    if (lane == 0) {
        if (!q_ok) {
            put(&p.bad[h.r], p.tag, 1u);
            __builtin_amdgcn_s_waitcnt(0);  // the mark is stored before the half word is published
        }
        put(&p.hw[h.sw], p.tag, u_bits);
    }
}

// A half word's union bits straight into the union plane (the bit planes are the refresh's whole
// result when no ids are asked for), and -1 as the request's count when q never arrived.
__device__ __forceinline__ void write_union_half(const RefreshParams& p, const HalfWord& h, unsigned u_bits, bool q_ok,
                                                 int lane) {
    if (lane == 0) {
        const int n_words_r = p.word_off[h.r + 1] - p.word_off[h.r];
        const size_t mw = (size_t)(p.n_idx + 1) * p.word_off[h.r] + (size_t)p.n_idx * n_words_r + h.lw;
        reinterpret_cast<unsigned*>(p.masks)[2 * mw + h.half] = u_bits;
        if (!q_ok) p.sel_count[h.r] = -1;
    }
}

// Score wave: half word sw (none when sw >= n_halves), all indexers in batches of U.
template <typename T, int DIDX>
__device__ void score_role(const RefreshParams& p, int sw) {
    using S = ScoreShape<T, DIDX>;
    const int lane = threadIdx.x & 63;
    if (sw >= p.n_halves) return;
    const HalfWord h = half_word<S::ROW>(p, sw);
    uint4 v[S::U][S::P];
    unsigned u_bits = 0u;
    bool q_ok = true;
    for (int i0 = 0; i0 < p.n_idx; i0 += S::U) {
        const int nu = min(S::U, p.n_idx - i0);
        load_runs<T, DIDX>(h, i0, nu, lane, v);
        asm volatile("" ::: "memory");  // every key load of the batch is issued before q is polled
        score_runs<T, DIDX>(p, h, i0, nu, lane, v, &u_bits, &q_ok);
    }
    if (p.bits_only)
        write_union_half(p, h, u_bits, q_ok, lane);
    else
        publish_half(p, h, u_bits, q_ok, lane);
}

// ------------------------------------------------------------------------------------------
// Compaction role: group c of a request handles the request's words [64c, 64c + 64) (its slice).
// All 256 threads read the union words up to the slice's end (thread t: words t, t+256, ...) until
// both halves of each carry this call's tag; the popcounts of the words before the slice give its base,
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
    const unsigned long long* hw = p.hw + (size_t)p.word_off[r] * 2;
    auto union_word = [&](int w, bool* ok) {
        // the union bits of the word's two halves, published by their score waves
        const unsigned long long lo = get(hw + 2 * (size_t)w), hi = get(hw + 2 * (size_t)w + 1);
        *ok = *ok && tagged(lo, p.tag) && tagged(hi, p.tag);
        return (unsigned long long)(unsigned)lo | ((unsigned long long)(unsigned)hi << 32);
    };
    // Runs of up to kKeep words per thread stay in registers: a word is read until all its units
    // carry this call's tag, then kept; requests longer than 256*kKeep words are re-read.
    constexpr int kKeep = 2;
    const bool held = s1 <= kThreads * kKeep;
    unsigned long long keep[kKeep] = {};
    unsigned done = 0u;
    bool failed = false;
    bool bad = false;
    for (unsigned spins = 0;; ++spins) {
        bool ok = true;
        if (held) {
            // both halves of every word this thread keeps, all requested at once (indices past the
            // slice's end clamped, their words ignored)
            unsigned long long lo[kKeep], hi[kKeep];
#pragma unroll
            for (int k = 0; k < kKeep; ++k) {
                const int w = min(t + kThreads * k, s1 - 1);
                lo[k] = get(hw + 2 * (size_t)w);
                hi[k] = get(hw + 2 * (size_t)w + 1);
            }
#pragma unroll
            for (int k = 0; k < kKeep; ++k) {
                const int w = t + kThreads * k;
                if (w < s1 && !((done >> k) & 1u)) {
                    if (tagged(lo[k], p.tag) && tagged(hi[k], p.tag)) {
                        keep[k] = (unsigned long long)(unsigned)lo[k] | ((unsigned long long)(unsigned)hi[k] << 32);
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
__global__ __launch_bounds__(kThreads, kGroupsPerCU) void refresh_kernel(RefreshParams p) {
    const int g = blockIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (g < p.n_encode_groups) {
        const int e = 4 * g + wave;
        if (e < p.n_encode_waves) encode_role<T>(p, e);
        return;
    }
    if (g < p.n_encode_groups + p.n_score_groups) {
        score_role<T, DIDX>(p, 4 * (g - p.n_encode_groups) + wave);
        return;
    }
    compact_role(p, g - p.n_encode_groups - p.n_score_groups);
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
    LSA_CHECK_ARG(a->select_level == 0.f || (a->select_level > 0.f && a->select_level < 1.f),
                  "lsa_index_refresh: select_level=%g (0 for 0.5, else strictly between 0 and 1)",
                  (double)a->select_level);
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
    off = align_up(off + (size_t)words * 2 * sizeof(unsigned long long), 256);
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
    rp.logits = a->logits;
    rp.bits_only = a->sel_ids == nullptr ? 1 : 0;
    for (int r = 0; r < a->n_req; ++r) rp.tslot[r] = a->table_out ? a->table_slot_base[r] : 0;
    rp.qw = reinterpret_cast<unsigned long long*>(ws + L.qw_off);
    rp.hw = reinterpret_cast<unsigned long long*>(ws + L.hw_off);
    rp.bad = reinterpret_cast<unsigned long long*>(ws + L.bad_off);
    rp.tag = (unsigned long long)call << 32;
    // the level's logit in double, then fp32 for the comparison with the fp32 logit (0 for 0.5)
    const double lev = a->select_level == 0.f ? 0.5 : (double)a->select_level;
    rp.select_logit = (float)std::log(lev / (1.0 - lev));
    rp.n_req = a->n_req;
    rp.d_model = a->d_model;
    rp.d_idx = a->d_idx;
    rp.n_idx = a->n_idx;
    rp.n_halves = L.total_words * 2;
    // encode waves: two W_q rows of one indexer for four requests each
    rp.n_encode_waves = a->n_idx * ((a->d_idx + kEncRows - 1) / kEncRows) * ((a->n_req + kEncReq - 1) / kEncReq);
    rp.n_encode_groups = (rp.n_encode_waves + kThreads / 64 - 1) / (kThreads / 64);
    rp.n_score_groups = (rp.n_halves + kThreads / 64 - 1) / (kThreads / 64);
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
    const dim3 grid(rp.n_encode_groups + rp.n_score_groups + (rp.bits_only ? 0 : co)), block(kThreads);
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
    LSA_CHECK_ARG(a->hidden && a->w_q && a->keys && a->bias && a->sel_count, "lsa_index_refresh: null device pointer");
    LSA_CHECK_ARG(a->sel_ids || (a->masks && !a->table_out),
                  "lsa_index_refresh: without sel_ids the refresh needs masks (its whole result) and no table_out");
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
    LSA_CHECK_ARG(((uintptr_t)a->logits % 4) == 0, "lsa_index_refresh: logits must be 4-byte aligned");
    const size_t eb = elem_bytes(a->dtype);
    LSA_CHECK_ARG(((uintptr_t)a->hidden % 16) == 0 && ((uintptr_t)a->w_q % 16) == 0 &&
                      ((uintptr_t)a->keys % 16) == 0 && ((uintptr_t)a->workspace % 256) == 0,
                  "lsa_index_refresh: hidden, w_q, keys must be 16-byte aligned and workspace 256-byte aligned");
    LSA_CHECK_ARG((a->hidden_req_stride * eb) % 16 == 0 && (a->hidden_idx_stride * eb) % 16 == 0,
                  "lsa_index_refresh: hidden strides must be multiples of 16 bytes");
    if (a->dtype == LSA_BF16) return launch_refresh<uint16_t>(a, L, stream);
    return launch_refresh<float>(a, L, stream);
}
