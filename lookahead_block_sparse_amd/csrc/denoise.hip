// Label denoising of the indexer's training labels (zhichai.net explainer of "FlashMemory-DeepSeek-
// V4", section 3 "Training the Indexer", the three-step pipeline): per CSA layer and token window,
// softmax over the window's history blocks and the smallest set of blocks whose probability reaches
// top_p; then, per window, the blocks at least min_votes layers keep.
//
// topp_kernel: one 256-thread group per (layer, window) row of up to 16,384 logits, held in
// registers (64 per thread, block b = thread + 256 k, so that element k of a wave is one 64-block
// word of the row's set and its ballot is that word).  Small groups keep several rows in flight on
// each compute unit: a row's steps are short chains of dependent work.  exp(x - max) is evaluated
// in fp64 (fixed48 below) and held as fixed point with 48 fraction bits, so the row's sums are exact
// and do not depend on the order of the additions, and "the running sum reaches top_p" is the integer test
// sum >= ceil(top_p * total).  Blocks are ranked by logit, equal logits by block id.  One pass
// builds a histogram of the mass over 2,048 logit buckets below the row's maximum (exact integer
// sums in LDS); a scan of the buckets gives the total and the bucket where the running mass reaches
// the target; every block of the buckets above it is kept, and the blocks of that bucket (usually a
// handful) are collected, given their exponentials, ranked against each other and walked in order
// until the target is met.  A bucket of more than 256 blocks (long runs of equal logits) falls
// back to a 32-step bisection on an order-preserving key: every block above the threshold key K is
// kept, and of the blocks at K (equal logits, equal probabilities) as many as the remaining mass
// needs, lowest ids first.
// vote_kernel: one group per window, one lane per 64-block word: a bit-sliced count of the layers'
// words, compared with min_votes bit by bit.
#include <hip/hip_ext.h>

#include <cmath>

#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 64;                      // logits per thread
constexpr int kMaxBlocks = kThreads * kPer;   // 16,384 blocks per row
constexpr int kVoteThreads = 256;
constexpr int kBuckets = 2048;   // logit buckets below the row maximum
constexpr int kBPerT = kBuckets / kThreads;
constexpr float kRange = 34.f;   // exp(-34) * 2^48 < 0.5: blocks further below the maximum carry no mass
constexpr int kCand = 256;       // largest boundary bucket ranked directly
constexpr int kBisThreads = 512; // crowded rows: 32 logits per thread
constexpr int kBisPer = 32;

struct TopPParams {
    const float* logits;
    long long stride;
    const int* n_blk;
    unsigned long long* sets;  // [n_layers][n_windows][words]
    int* crowded;              // [n_layers * n_windows]: 1 when the row's boundary bucket is crowded
    unsigned long long mant;   // top_p = mant * 2^-shift
    int shift;
    int n_windows, words;
};

struct VoteParams {
    const unsigned long long* sets;
    unsigned long long* labels;
    int* n_pos;
    int* n_naive;
    int n_layers, n_windows, words, min_votes;
};

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned lo = __shfl_xor((unsigned)v, o, 64), hi = __shfl_xor((unsigned)(v >> 32), o, 64);
        v += ((unsigned long long)hi << 32) | lo;
    }
    return v;
}

// larger logit -> larger key; -0 is folded into +0 by the caller
__device__ __forceinline__ unsigned order_key(float x) {
    const unsigned u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// round(2^48 exp(d)) for d <= 0 (round to nearest, ties to even), by Tang's table-driven method
// (P. T. P. Tang, ACM TOMS 15(2), 1989): d = t ln2/32 + r with t = rint(32 d / ln 2) and
// |r| <= ln2/64, exp(d) = 2^(t >> 5) 2^((t & 31)/32) exp(r), exp(r) by its Taylor polynomial of
// degree 6 (truncation below 4e-18 relative on that range), 2^(j/32) from a 32-entry table.
// ln2/32 is split into a 42-bit head, whose products with |t| < 2^11 are exact, and the rest.
// d is clamped at -40 first: 2^48 exp(-40) < 0.5 rounds to 0, as does -inf.  Adding 2^52 to the
// result, a value in [0, 2^48], leaves its rounded integer in the low mantissa bits.
__device__ __forceinline__ unsigned long long fixed48(double d, const double* pow2_32nd) {
    constexpr double kInvStep = 0x1.71547652b82fep+5;  // 32 / ln 2
    constexpr double kStepHi = 0x1.62e42fefa3800p-6;   // ln 2 / 32, high 42 bits
    constexpr double kStepLo = 0x1.ef35793c76730p-50;  // ln 2 / 32 - kStepHi
    d = fmax(d, -40.0);
    const double t = rint(d * kInvStep);
    const int n = (int)t;  // in [-1847, 0]
    const double r = fma(-t, kStepLo, fma(-t, kStepHi, d));
    double q = fma(r, 1.0 / 720.0, 1.0 / 120.0);
    q = fma(r, q, 1.0 / 24.0);
    q = fma(r, q, 1.0 / 6.0);
    q = fma(r, q, 0.5);
    q = fma(r, q, 1.0);
    q = fma(r, q, 1.0);
    const double y = ldexp(pow2_32nd[n & 31] * q, (n >> 5) + 48) + 4503599627370496.0;
    return (unsigned long long)__double_as_longlong(y) - 0x4330000000000000ull;
}

// The logits' registers as if rewritten: each pass recomputes what it derives from them (bucket,
// key) instead of the compiler keeping a second register per logit live across passes.
template <int N>
__device__ __forceinline__ void opaque(float (&v)[N]) {
#pragma unroll
    for (int k = 0; k < N; ++k) asm volatile("" : "+v"(v[k]));
}

// 64-bit inclusive scan across the wave
__device__ __forceinline__ unsigned long long wave_scan_u64(unsigned long long v, int lane) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned lo = __shfl_up((unsigned)v, o, 64), hi = __shfl_up((unsigned)(v >> 32), o, 64);
        if (lane >= o) v += ((unsigned long long)hi << 32) | lo;
    }
    return v;
}

__global__ __launch_bounds__(kThreads) void topp_kernel(TopPParams p) {
    __shared__ unsigned long long s_hmass[kBuckets];
    __shared__ double s_pow2[32];               // 2^(j/32)
    __shared__ unsigned long long s_kw[kMaxBlocks / 64];  // boundary-bucket blocks kept: set words
    __shared__ unsigned s_ck[kCand];
    __shared__ int s_cid[kCand];
    __shared__ float s_cx[kCand];
    __shared__ unsigned long long s_se[kCand];
    __shared__ int s_crank[kCand];
    __shared__ unsigned long long s_wsum[kWaves];
    __shared__ float s_max[kWaves];
    __shared__ int s_bstar, s_pstar;
    __shared__ unsigned long long s_before;
    __shared__ unsigned s_nc, s_kmax;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = blockIdx.x;  // layer * n_windows + window
    const int n = p.n_blk[row % p.n_windows];
    const float* x = p.logits + (size_t)row * p.stride;

    for (int k = threadIdx.x; k < kBuckets; k += kThreads) s_hmass[k] = 0ull;
    for (int k = threadIdx.x; k < kMaxBlocks / 64; k += kThreads) s_kw[k] = 0ull;
    if (threadIdx.x == 0) {
        s_nc = 0u;
        s_kmax = 0u;
    }
    if (threadIdx.x < 32) s_pow2[threadIdx.x] = exp2((double)threadIdx.x / 32.0);

    // unconditional loads, all in flight at once, through a buffer resource over the row: one
    // offset register, a scalar offset per load, and zeros (not memory) past the row's end
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(x), (short)0, n * (int)sizeof(float), 0x00020000);
    float xv[kPer];
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        xv[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)threadIdx.x * 4, kThreads * 4 * k, 0));
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        float v = (int)threadIdx.x + kThreads * k < n ? xv[k] : -INFINITY;
        if (v == 0.f) v = 0.f;  // -0 and +0 are the same logit
        xv[k] = v;
        mx = fmaxf(mx, v);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) s_max[wave] = mx;
    __syncthreads();  // also orders the clears and the table before the histogram
#pragma unroll
    for (int k = 0; k < kWaves; ++k) mx = fmaxf(mx, s_max[k]);

    // (max - v) 2048/34 in one fused multiply-add, truncated, the far blocks in the last bucket:
    // monotone in the logit (a rounded fma is), so equal logits share a bucket and a higher logit
    // never lands in a later bucket; the row's maximum (a result in (-1, 1)) is in bucket 0
    constexpr float kScale = (float)kBuckets / kRange;
    const float mx_s = mx * kScale;
    auto bucket_of = [&](float v) { return (int)fminf(fmaf(-v, kScale, mx_s), (float)(kBuckets - 1)); };
    // probabilities up to the common factor 1/total (not kept: the boundary bucket's blocks
    // recompute theirs once collected)
    auto fixed_e = [&](float v) { return fixed48((double)v - (double)mx, s_pow2); };

    // ---- mass histogram over logit buckets below the maximum (exact sums: integer LDS atomics) ----
    // Blocks past the row's end hold -inf, like a real logit of -inf: no mass, the last bucket,
    // ranked below every other block of that bucket (ties by id, and their ids are the largest),
    // hence never kept; the steps below need no bounds test.
#pragma unroll
    for (int k = 0; k < kPer; ++k) atomicAdd(&s_hmass[bucket_of(xv[k])], fixed_e(xv[k]));
    opaque(xv);
    __syncthreads();
    // the row's total and the bucket where the running mass (highest logits first) reaches the
    // target: thread t owns buckets kBPerT t .. kBPerT t + kBPerT - 1; an exclusive scan of the
    // owners' sums locates it, and the last inclusive sum is the total
    {
        unsigned long long own = 0;
#pragma unroll
        for (int q = 0; q < kBPerT; ++q) own += s_hmass[kBPerT * threadIdx.x + q];
        const unsigned long long inc = wave_scan_u64(own, lane);
        if (lane == 63) s_wsum[wave] = inc;
        __syncthreads();
        unsigned long long run = inc - own, total = 0;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            total += s_wsum[v];
            run += v < wave ? s_wsum[v] : 0ull;
        }
        // target = ceil(top_p * total), exactly: top_p = mant / 2^shift
        const unsigned __int128 prod = (unsigned __int128)p.mant * total;
        const unsigned long long target =
            (unsigned long long)((prod + (((unsigned __int128)1 << p.shift) - 1)) >> p.shift);
#pragma unroll
        for (int q = 0; q < kBPerT; ++q) {
            const unsigned long long m = s_hmass[kBPerT * threadIdx.x + q];
            if (run < target && run + m >= target) {
                s_bstar = kBPerT * threadIdx.x + q;
                s_before = target - run;  // the mass still needed from the boundary bucket
            }
            run += m;
        }
    }
    __syncthreads();
    const int bstar = s_bstar;
    const unsigned long long need_b = s_before;  // > 0, <= the bucket's mass
    // The boundary bucket's blocks: key, id and logit, and their largest key.  Its blocks lie in
    // [max - (bstar + 1) / scale, max - bstar / scale] up to the rounding of the bucket's fma (a few
    // fp32 units of the logits' magnitude, far inside the slack below); only the blocks of that
    // widened interval take the exact test.
    const float slack = 0x1p-12f * (1.0f + fabsf(mx));
    const float lo = bstar == kBuckets - 1 ? -INFINITY : mx - (float)(bstar + 1) / kScale - slack;
    const float hi = mx - (float)bstar / kScale + slack;
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));  // block ids recomputed per pass, not kept from the loads
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int b = tid + kThreads * k;
        if (xv[k] >= lo && xv[k] <= hi && bucket_of(xv[k]) == bstar) {
            const unsigned pos = atomicAdd(&s_nc, 1u);
            const unsigned key = order_key(xv[k]);
            atomicMax(&s_kmax, key);
            if (pos < (unsigned)kCand) {
                s_ck[pos] = key;
                s_cid[pos] = b;
                s_cx[pos] = xv[k];
            }
        }
    }
    opaque(xv);
    __syncthreads();
    const unsigned cb = s_nc;
    if (cb > (unsigned)kCand) {  // long runs of equal logits: topp_bisect_kernel takes the row
        if (threadIdx.x == 0) p.crowded[row] = 1;
        return;
    }
    if (threadIdx.x == 0) p.crowded[row] = 0;
    // ranked by (logit desc, id asc), walked until the target; the ones kept are marked in s_kw
    auto mark = [&](int id) { atomicOr(&s_kw[id >> 6], 1ull << (id & 63)); };
    if (cb <= 64) {
        // usually a few dozen blocks: one wave holds them (lane c: candidate c), ranks them against
        // each other's lanes, scans their masses in rank order and marks the kept ones, with no
        // group-wide barrier
        if (wave == 0) {
            const int c = lane;
            const unsigned kc = c < (int)cb ? s_ck[c] : 0u;
            const int id = c < (int)cb ? s_cid[c] : 0;
            int rank = 0;
            for (int q = 0; q < (int)cb; ++q) {  // q uniform: lane q's values read into scalars
                const unsigned kq = (unsigned)__builtin_amdgcn_readlane((int)kc, q);
                const int iq = __builtin_amdgcn_readlane(id, q);
                rank += (kq > kc) | ((kq == kc) & (iq < id));
            }
            if (c < (int)cb) s_se[rank] = fixed_e(s_cx[c]);
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            const unsigned long long own = lane < (int)cb ? s_se[lane] : 0ull;  // mass of rank `lane`
            const unsigned long long inc = wave_scan_u64(own, lane);
            // the first rank whose running mass reaches need_b
            const unsigned long long hit = __ballot(lane < (int)cb && inc >= need_b && inc - own < need_b);
            const int pstar = hit ? __builtin_ctzll(hit) : (int)cb - 1;
            if (c < (int)cb && rank <= pstar) mark(id);
        }
    } else {
        // one rank per thread
        const int c = threadIdx.x;
        int rank = 0;
        if (c < (int)cb) {
            const unsigned kc = s_ck[c];
            const int ic = s_cid[c];
            for (int q = 0; q < (int)cb; ++q) rank += (s_ck[q] > kc || (s_ck[q] == kc && s_cid[q] < ic)) ? 1 : 0;
            s_se[rank] = fixed_e(s_cx[c]);
            s_crank[c] = rank;
        }
        __syncthreads();
        const unsigned long long own = c < (int)cb ? s_se[c] : 0ull;  // mass of rank c
        const unsigned long long inc = wave_scan_u64(own, lane);
        if (lane == 63) s_wsum[wave] = inc;  // the bucket scan's reads of s_wsum ended two barriers ago
        __syncthreads();
        unsigned long long run = inc - own;
        for (int v = 0; v < wave; ++v) run += s_wsum[v];
        if (c < (int)cb && run < need_b && run + own >= need_b) s_pstar = c;
        __syncthreads();
        const int pstar = s_pstar;
        if (c < (int)cb && s_crank[c] <= pstar) mark(s_cid[c]);
    }
    __syncthreads();
    // Blocks of the buckets above the boundary bucket have larger logits than every block of it
    // (bucket_of is monotone), so they are the blocks above its largest logit; with the marked
    // blocks of the boundary bucket they are the set.  Element k of the wave is word kWaves k + wave
    // of the set: lane k holds that word for the store (one coalesced store per lane).
    const unsigned km = s_kmax;
    const float cmax = __uint_as_float((km & 0x80000000u) ? (km & 0x7fffffffu) : ~km);  // order_key inverted
    unsigned long long myword = 0ull;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const unsigned long long bits = __ballot(xv[k] > cmax);
        myword = lane == k ? bits : myword;
    }
    const int word = kWaves * lane + wave;
    myword |= s_kw[word];
    if (word < p.words) p.sets[(size_t)row * p.words + word] = myword;
}


// Rows whose boundary bucket is crowded (flagged by topp_kernel): a 32-step bisection on the key.
__global__ __launch_bounds__(kBisThreads) void topp_bisect_kernel(TopPParams p) {
    if (p.crowded[blockIdx.x] == 0) return;
    constexpr int kThreads = kBisThreads, kWaves = kBisThreads / 64, kPer = kBisPer;
    __shared__ unsigned long long s_red[2][kWaves];
    __shared__ float s_max[kWaves];
    __shared__ int s_cnt[kPer][kWaves];
    __shared__ double s_pow2[32];  // 2^(j/32)
    if (threadIdx.x < 32) s_pow2[threadIdx.x] = exp2((double)threadIdx.x / 32.0);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = blockIdx.x;  // layer * n_windows + window
    const int n = p.n_blk[row % p.n_windows];
    const float* x = p.logits + (size_t)row * p.stride;

    int parity = 0;
    // block-wide exact sum: two LDS buffers in turn, so one barrier per sum
    auto block_sum = [&](unsigned long long v) {
        v = wave_sum_u64(v);
        if (lane == 0) s_red[parity][wave] = v;
        __syncthreads();
        unsigned long long t = 0;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) t += s_red[parity][k];
        parity ^= 1;
        return t;
    };

    float xv[kPer];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int b = threadIdx.x + kThreads * i;
        float v = b < n ? x[b] : -INFINITY;
        if (v == 0.f) v = 0.f;  // -0 and +0 are the same logit
        xv[i] = v;
        mx = fmaxf(mx, v);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) s_max[wave] = mx;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kWaves; ++k) mx = fmaxf(mx, s_max[k]);

    // probabilities up to the common factor 1/total: exp(x - max) in fp64, 48 fraction bits
    unsigned long long e[kPer];
    unsigned key[kPer];
    unsigned long long part = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int b = threadIdx.x + kThreads * i;
        if (b < n) {
            e[i] = fixed48((double)xv[i] - (double)mx, s_pow2);
            key[i] = order_key(xv[i]);
        } else {
            e[i] = 0ull;
            key[i] = 0u;  // below every real logit's key (-inf maps to 0x007fffff)
        }
        part += e[i];
    }
    const unsigned long long total = block_sum(part);
    // target = ceil(top_p * total), exactly: top_p = mant / 2^shift
    const unsigned __int128 prod = (unsigned __int128)p.mant * total;
    const unsigned long long target =
        (unsigned long long)((prod + (((unsigned __int128)1 << p.shift) - 1)) >> p.shift);

    // the largest key K whose blocks at or above it carry at least the target
    unsigned K = 0u;
    for (int bit = 31; bit >= 0; --bit) {
        const unsigned cand = K | (1u << bit);
        unsigned long long s = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) s += key[i] >= cand ? e[i] : 0ull;
        if (block_sum(s) >= target) K = cand;
    }
    // mass strictly above K, and the blocks at K (equal logits: equal probabilities)
    unsigned long long above = 0, n_tie = 0, tie_sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        above += key[i] > K ? e[i] : 0ull;
        n_tie += key[i] == K ? 1ull : 0ull;
        tie_sum += key[i] == K ? e[i] : 0ull;
    }
    above = block_sum(above);
    n_tie = block_sum(n_tie);
    tie_sum = block_sum(tie_sum);
    // the tied blocks share one logit, hence one value: the sum over them / their number is exact
    const unsigned long long ek = tie_sum / n_tie;             // > 0: the tied blocks carry mass
    const unsigned long long need = (target - above + ek - 1) / ek;  // tied blocks to keep, <= n_tie

    // ranks of the tied blocks in block-id order (only when some of them stay out): tied blocks per
    // (i, wave) slice, then an exclusive prefix over the slices in id order
    const bool partial = need < n_tie;
    if (partial) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const unsigned long long tb = __ballot(key[i] == K);
            if (lane == 0) s_cnt[i][wave] = __popcll(tb);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            int run = 0;
            for (int i = 0; i < kPer; ++i)
                for (int v = 0; v < kWaves; ++v) {
                    const int c = s_cnt[i][v];
                    s_cnt[i][v] = run;
                    run += c;
                }
        }
        __syncthreads();
    }
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        bool keep = key[i] > K;
        const unsigned long long tb = __ballot(key[i] == K);
        if (key[i] == K)
            keep = !partial || (unsigned long long)(s_cnt[i][wave] + __popcll(tb & below)) < need;
        const unsigned long long bits = __ballot(keep);
        const int word = kWaves * i + wave;
        if (lane == 0 && word < p.words) p.sets[(size_t)row * p.words + word] = bits;
    }
}

// One group per window, one lane per 64-block word of it: the lane adds its word of every layer into
// a bit-sliced counter (bit b of plane c[k] is bit k of block b's count; ripple-carry adds of one-bit
// values, 7 planes count up to 64 layers), then compares the counts with min_votes plane by plane.
// Loads of consecutive lanes are consecutive words (coalesced); the window's counts are reduced in
// LDS (no atomics: the counters of all windows share a few cache lines, where device atomics
// serialize).
__global__ __launch_bounds__(kVoteThreads) void vote_kernel(VoteParams p) {
    __shared__ int s_pos[kVoteThreads / 64], s_naive[kVoteThreads / 64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int w = blockIdx.x;
    int pos = 0, naive = 0;
    for (int word = threadIdx.x; word < p.words; word += kVoteThreads) {
        unsigned long long c[7] = {0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull};
        unsigned long long any = 0ull;
        for (int l = 0; l < p.n_layers; ++l) {
            const unsigned long long x = p.sets[((size_t)l * p.n_windows + w) * p.words + word];
            any |= x;
            unsigned long long carry = x;
#pragma unroll
            for (int k = 0; k < 7; ++k) {
                const unsigned long long t = c[k] & carry;
                c[k] ^= carry;
                carry = t;
            }
        }
        // count >= min_votes, per bit, from the most significant plane down
        unsigned long long gt = 0ull, eq = ~0ull;
#pragma unroll
        for (int k = 6; k >= 0; --k) {
            const unsigned long long mk = ((p.min_votes >> k) & 1) ? ~0ull : 0ull;
            gt |= eq & c[k] & ~mk;
            eq &= ~(c[k] ^ mk);
        }
        const unsigned long long lab = gt | eq;
        p.labels[(size_t)w * p.words + word] = lab;
        pos += __popcll(lab);
        naive += __popcll(any);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        pos += __shfl_xor(pos, o, 64);
        naive += __shfl_xor(naive, o, 64);
    }
    if (lane == 0) {
        s_pos[wave] = pos;
        s_naive[wave] = naive;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int a = 0, b = 0;
        for (int k = 0; k < kVoteThreads / 64; ++k) {
            a += s_pos[k];
            b += s_naive[k];
        }
        p.n_pos[w] = a;
        if (p.n_naive) p.n_naive[w] = b;
    }
}

struct DenoisePlan {
    int words = 0;
    size_t sets_bytes = 0;   // layer sets, when the caller does not take them
    size_t flags_off = 0;    // crowded-row flags in the workspace
    size_t total = 0;        // workspace bytes
};

lsa_status denoise_plan(const lsa_denoise_args* a, DenoisePlan* P) {
    LSA_CHECK_ARG(a != nullptr, "lsa_label_denoise: null args");
    LSA_CHECK_ARG(a->n_layers >= 1 && a->n_layers <= 64, "lsa_label_denoise: n_layers=%d outside 1..64", a->n_layers);
    LSA_CHECK_ARG(a->n_windows >= 1 && a->n_windows <= 65536, "lsa_label_denoise: n_windows=%d outside 1..65536",
                  a->n_windows);
    LSA_CHECK_ARG(a->min_votes >= 1 && a->min_votes <= a->n_layers, "lsa_label_denoise: min_votes=%d outside 1..%d",
                  a->min_votes, a->n_layers);
    LSA_CHECK_ARG(a->reserved0 == 0, "lsa_label_denoise: reserved0 must be 0");
    LSA_CHECK_ARG(a->top_p > 0.0 && a->top_p <= 1.0 && a->top_p >= std::ldexp(1.0, -30),
                  "lsa_label_denoise: top_p=%g outside [2^-30, 1]", a->top_p);
    LSA_CHECK_ARG(a->n_blk != nullptr, "lsa_label_denoise: n_blk is null");
    int mx = 0;
    for (int w = 0; w < a->n_windows; ++w) {
        LSA_CHECK_SUP(a->n_blk[w] >= 1 && a->n_blk[w] <= kMaxBlocks,
                      "lsa_label_denoise: window %d has %d blocks (1..%d)", w, a->n_blk[w], kMaxBlocks);
        mx = std::max(mx, a->n_blk[w]);
    }
    LSA_CHECK_ARG(a->logit_stride >= mx, "lsa_label_denoise: logit_stride=%lld < %d blocks",
                  (long long)a->logit_stride, mx);
    P->words = (mx + 63) / 64;
    P->sets_bytes = (size_t)a->n_layers * a->n_windows * P->words * sizeof(unsigned long long);
    P->flags_off = a->layer_sets ? 0 : align_up(P->sets_bytes, 256);
    P->total = P->flags_off + (size_t)a->n_layers * a->n_windows * sizeof(int);
    return LSA_OK;
}

}  // namespace
}  // namespace lsa

using namespace lsa;

extern "C" lsa_status lsa_label_denoise_workspace(const lsa_denoise_args* a, size_t* bytes) {
    DenoisePlan P;
    lsa_status st = denoise_plan(a, &P);
    if (st != LSA_OK) return st;
    LSA_CHECK_ARG(bytes != nullptr, "lsa_label_denoise_workspace: bytes is null");
    *bytes = P.total;
    return LSA_OK;
}

extern "C" lsa_status lsa_label_denoise(const lsa_denoise_args* a, hipStream_t stream) {
    DenoisePlan P;
    lsa_status st = denoise_plan(a, &P);
    if (st != LSA_OK) return st;
    LSA_CHECK_ARG(a->logits && a->n_blk_dev && a->labels && a->n_pos, "lsa_label_denoise: null device pointer");
    LSA_CHECK_ARG(((uintptr_t)a->logits % 4) == 0 && ((uintptr_t)a->labels % 8) == 0 &&
                      (a->layer_sets == nullptr || ((uintptr_t)a->layer_sets % 8) == 0),
                  "lsa_label_denoise: misaligned logits, labels or layer_sets");
    if (a->workspace == nullptr || a->workspace_bytes < P.total)
        return fail(LSA_ERR_WORKSPACE, "lsa_label_denoise: workspace of %zu bytes, need %zu",
                    a->workspace ? a->workspace_bytes : (size_t)0, P.total);
    LSA_CHECK_ARG(((uintptr_t)a->workspace % 8) == 0, "lsa_label_denoise: misaligned workspace");
    unsigned long long* sets = reinterpret_cast<unsigned long long*>(a->layer_sets);
    if (sets == nullptr) sets = static_cast<unsigned long long*>(a->workspace);
    TopPParams tp;
    tp.logits = a->logits;
    tp.stride = a->logit_stride;
    tp.n_blk = a->n_blk_dev;
    tp.sets = sets;
    tp.crowded = reinterpret_cast<int*>(static_cast<char*>(a->workspace) + P.flags_off);
    int ex = 0;
    const double f = std::frexp(a->top_p, &ex);  // top_p = f 2^ex, f in [0.5, 1)
    tp.mant = (unsigned long long)std::ldexp(f, 53);
    tp.shift = 53 - ex;
    tp.n_windows = a->n_windows;
    tp.words = P.words;
    const dim3 grid(a->n_layers * a->n_windows), block(kThreads);
    if (a->ev_begin && a->ev_end)  // the events take the dispatch's own start and end timestamps
        hipExtLaunchKernelGGL(topp_kernel, grid, block, 0, stream, a->ev_begin, a->ev_end, 0, tp);
    else
        hipLaunchKernelGGL(topp_kernel, grid, block, 0, stream, tp);
    LSA_HIP(hipGetLastError());
    hipLaunchKernelGGL(topp_bisect_kernel, grid, dim3(kBisThreads), 0, stream, tp);
    LSA_HIP(hipGetLastError());
    VoteParams vp;
    vp.sets = sets;
    vp.labels = reinterpret_cast<unsigned long long*>(a->labels);
    vp.n_pos = a->n_pos;
    vp.n_naive = a->n_naive;
    vp.n_layers = a->n_layers;
    vp.n_windows = a->n_windows;
    vp.words = P.words;
    vp.min_votes = a->min_votes;
    hipLaunchKernelGGL(vote_kernel, dim3(a->n_windows), dim3(kVoteThreads), 0, stream, vp);
    LSA_HIP(hipGetLastError());
    return LSA_OK;
}
