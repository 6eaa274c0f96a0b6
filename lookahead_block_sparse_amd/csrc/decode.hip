// Block-sparse flash-decode over the recent window and the loaded blocks (zhichai.net explainer of
// "FlashMemory-DeepSeek-V4", section 2 step 4: the decode steps attend only over the loaded blocks;
// section 1: the recent window).
//
// Work unit: a tile = one 64-token block (a hot-pool slot or a window-ring block).  Request r has
// n_sel[r] block tiles (its table, ascending block id) followed by the ring tiles that hold window
// tokens.  The tiles of all requests are concatenated and cut into G equal contiguous ranges, one per
// work-group (split-K, balanced whatever the request mix), one group of 8 waves per compute unit.
// Inside a group the waves take the tiles of each request segment on demand from a counter in LDS and
// keep their own online-softmax state; at the end of a segment the waves are combined in LDS and the
// group writes one partial (m, l, o) per segment.  The merge kernel combines a request's partials by
// log-sum-exp.  (The wave scheduler favours the oldest waves, so waves of one unit progress at very
// different rates; taking tiles on demand lets the fast ones take more.)
//
// Matrix cores (bf16): per tile and wave, S^T = K Q^T is 16 v_mfma_f32_16x16x32_bf16 (rows = tokens,
// columns = the 16 query heads) and O^T += V^T P^T another 16.  The token order inside each S^T
// sub-tile is chosen so that the S^T accumulator a lane holds is exactly the P operand it feeds to the
// V^T P^T product (no cross-lane movement of P).  bf16 blocks are stored in that fragment order, so
// each operand is one 16-byte load per lane and the 64 lanes of a load read 1 KiB of whole cache lines
// (half-line reads, as a row-major block gives, cost about a tenth of the read bandwidth).  fp32
// inputs use v_mfma_f32_16x16x4_f32 with the same accumulator layout on row-major K and V^T.
#include <hip/hip_ext.h>

#include <cmath>
#include <mutex>
#include <vector>

#include "lsa_internal.hpp"

namespace lsa {
namespace {

constexpr int kMaxReq = LSA_MAX_DECODE_REQ;
constexpr int kWaves = 8;  // one work-group per CU: its waves share the segment's tiles
constexpr int kThreads = 64 * kWaves;
constexpr int kStage = 1024;  // table entries staged in LDS at a time
constexpr int kHeads = 16;  // query heads per MFMA column block (n_heads <= 16 padded with zeros)

struct DecodeParams {
    const void* q;
    const void* k_new;
    const void* v_new;
    char* ring;
    long long ring_req_bytes;
    const char* pool;
    const int2* table;
    float* part_o;   // [P][16][D]
    float* part_ml;  // [P][16][2]
    int* mrange;     // device-side counts: [n_req][2] first and last group of each request, for the merge
    const int* n_sel_dev;  // optional: entry counts on the device (n_sel then holds capacities)
    int n_req, n_heads, n_chunks, win_cap, n_slots, n_groups;
    float scale_log2;
    int seq_len[kMaxReq];
    int ws[kMaxReq];
    int tbl_off[kMaxReq];
    int n_sel[kMaxReq];
    int n_ring[kMaxReq];  // window tiles of each request
    int ring_first[kMaxReq];
    int tile_prefix[kMaxReq + 1];  // host-side counts: the split computed on the host
    int row[kMaxReq];  // request r's row in q, k_new, v_new, ring and n_sel_dev
};

struct MergeParams {
    const float* part_o;
    const float* part_ml;
    const int* mrange;  // device-side counts: each request's groups, written by the attention kernel
    float* out;
    const int* n_sel_dev;
    int n_req, n_heads, n_groups;
    int n_sel[kMaxReq];
    int n_ring[kMaxReq];
    int w_lo[kMaxReq];  // host-side counts: the groups of each request, computed on the host
    int w_hi[kMaxReq];
    int row[kMaxReq];  // request r's row in out
};

// With device-side counts, the split of the tiles over the groups is computed by every group of both
// kernels from the same inputs (with host-side counts the host computes it): request r's tiles are
// [pre[r], pre[r+1]) of T = pre[n_req] (its n_sel[r] block tiles, read from the device when the
// counts live there, then its window tiles), split over split_groups(launched groups, T) groups.
__device__ void tile_split(const int* n_sel_dev, const int* n_sel, const int* n_ring, const int* row, int n_req,
                           int* s_ns, int* s_pre) {
    if ((int)threadIdx.x < n_req) {
        int ns = n_sel[threadIdx.x];
        if (n_sel_dev) ns = min(max(n_sel_dev[row[threadIdx.x]], 0), ns);
        s_ns[threadIdx.x] = ns;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int pre = 0;
        for (int r = 0; r < n_req; ++r) {
            s_pre[r] = pre;
            pre += s_ns[r] + n_ring[r];
        }
        s_pre[n_req] = pre;
    }
    __syncthreads();
}

// XCD-aware split.  Work-groups go to the 8 XCDs round-robin (group w runs on XCD w mod 8), and the
// odd-numbered XCDs read HBM measurably slower than the even ones: with equal shares, per-group
// timestamps show the groups on odd XCDs finishing 3-6 us after the others in a ~66 us launch.  So a
// group on an odd XCD gets kOddWeight/kEvenWeight of the tiles of a group on an even one (90% was
// the best of 85-100% measured; it shortens the launch by ~1 us).  Group w takes tiles
// [split_bound(w), split_bound(w + 1)); with T >= 2 G every group has at least one tile.
constexpr long long kEvenWeight = 100, kOddWeight = 90;
__host__ __device__ __forceinline__ long long split_prefix(long long w) {
    return kEvenWeight * w - (kEvenWeight - kOddWeight) * (w / 2);
}
__host__ __device__ __forceinline__ long long split_bound(long long w, long long T, long long G) {
    return T * split_prefix(w) / split_prefix(G);
}
// groups used for T tiles when the host does not know T: at most n_groups, and T >= 2 G
__host__ __device__ __forceinline__ long long split_groups(long long n_groups, long long T) {
    return T / 2 < n_groups ? (T / 2 > 1 ? T / 2 : 1) : n_groups;
}
// the group whose range holds tile x (0 <= x < T): the largest w with split_bound(w) <= x, where
// floor(T P(w) / P(G)) <= x  <=>  T P(w) < (x + 1) P(G): products only (a 64-bit division is a
// long instruction sequence on the GPU, and the search makes eight of them)
__device__ __forceinline__ int split_group_of(long long x, long long T, long long G) {
    const long long rhs = (x + 1) * split_prefix(G);
    int lo = 0, hi = (int)G - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (T * split_prefix(mid) < rhs) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------------------------------
// bf16 operands.  Lane l: lr = l % 16, lg = l / 16.
//   S^T sub-tile j (16 tokens), k-step ks: A = K[token][32ks + 8lg .. +8], token = tokK(j, lr)
//   accumulator element i of sub-tile j is token tokC(j, lg, i)
//   O^T += V^T P^T, k-step kk (32 tokens), d-tile dt: A = Vt[16dt + lr][32kk + 8lg .. +8],
//   B = P[h = lr][32kk + 8lg .. +8] = the lane's own accumulator values of sub-tiles 2kk, 2kk+1.
template <int D>
struct Bf16Ops {
    static constexpr int KS = D / 32;
    static constexpr int DT = D / 16;
    static constexpr int EB = 2;
    struct Frag {
        bf16x8 k[4][KS];
        bf16x8 v[DT][2];
    };
    struct QReg {
        bf16x8 b[KS];
    };
    __device__ static int tokK(int j, int lr) { return 32 * (j >> 1) + 8 * (lr >> 2) + 4 * (j & 1) + (lr & 3); }
    __device__ static int tokC(int j, int lg, int i) { return 32 * (j >> 1) + 8 * lg + 4 * (j & 1) + i; }

    __device__ static void load_q(QReg& q, const uint16_t* qr, int n_heads, int lane) {
        const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (lr < n_heads)
                q.b[ks] = *reinterpret_cast<const bf16x8*>(qr + lr * D + 32 * ks + 8 * lg);
            else
                q.b[ks] = bf16x8{};
        }
    }
    // The block is stored in fragment order: operand (j, ks) of K and (dt, kk) of V^T are each 1 KiB
    // of 16-byte pieces in lane order, so every load instruction reads whole cache lines.  The loads
    // are non-temporal: the tile is used once per launch.
    __device__ static void load(Frag& f, const char* base, int lane) {
        const bf16x8* kp = reinterpret_cast<const bf16x8*>(base) + lane;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) f.k[j][ks] = __builtin_nontemporal_load(kp + (j * KS + ks) * 64);
        const bf16x8* vp = reinterpret_cast<const bf16x8*>(base + 64 * D * EB) + lane;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) f.v[dt][kk] = __builtin_nontemporal_load(vp + (dt * 2 + kk) * 64);
    }
    // Issue point of a tile: every load of the tile (K then V) stays before this point and only the
    // K operands must have arrived, so the V loads are still in flight during Q K^T.
    __device__ static void pin_k(const Frag& f) {
        if constexpr (KS == 4) {
            asm volatile("" :: "v"(f.k[0][0]), "v"(f.k[0][1]), "v"(f.k[0][2]), "v"(f.k[0][3]), "v"(f.k[1][0]), "v"(f.k[1][1]), "v"(f.k[1][2]), "v"(f.k[1][3]), "v"(f.k[2][0]), "v"(f.k[2][1]), "v"(f.k[2][2]), "v"(f.k[2][3]), "v"(f.k[3][0]), "v"(f.k[3][1]), "v"(f.k[3][2]), "v"(f.k[3][3]) : "memory");
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) asm volatile("" :: "v"(f.k[j][ks]) : "memory");
        }
    }
    // Partial dot product of this lane's query elements (head lr, dims 32ks + 8lg + e) with k_new.
    __device__ static float dot_q_new(const QReg& q, const uint16_t* kn, int lane) {
        const int lg = lane >> 4;
        float acc = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 k = *reinterpret_cast<const bf16x8*>(kn + 32 * ks + 8 * lg);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf((float)q.b[ks][e], (float)k[e], acc);
        }
        return acc;
    }
    // v_new[16dt + 4lg + i]: the value entries of the output elements this lane accumulates.
    __device__ static void load_vnew(const uint16_t* vn, int lane, float v[DT][4]) {
        const int lg = lane >> 4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const uint2 w = *reinterpret_cast<const uint2*>(vn + 16 * dt + 4 * lg);
            v[dt][0] = bf16_lo(w.x);
            v[dt][1] = bf16_hi(w.x);
            v[dt][2] = bf16_lo(w.y);
            v[dt][3] = bf16_hi(w.y);
        }
    }
    __device__ static void qk(const Frag& f, const QReg& q, f32x4 s[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.k[j][ks], q.b[ks], acc, 0, 0, 0);
            s[j] = acc;
        }
    }
    __device__ static void pv(const Frag& f, const float p[16], f32x4 o[DT]) {
        bf16x8 pb[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[kk][e] = (__bf16)p[8 * kk + e];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.v[dt][kk], pb[kk], o[dt], 0, 0, 0);
    }
    // Store the current token into ring row `cur` (K row and V^T column).
    // Row t of the block (fragment order): the key's 8-element piece d/8 sits in operand
    // (j, ks = d/32) at lane u + 16 (d/8 % 4); the value of dimension d is element t % 8 of the piece
    // of operand (d/16, t/32) at lane d % 16 + 16 (t/8 % 4).
    __device__ static void write_current(char* base, int t, const uint16_t* kn, const uint16_t* vn, int lane) {
        uint16_t* b = reinterpret_cast<uint16_t*>(base);
        const int j = 2 * (t >> 5) + ((t >> 2) & 1), u = 4 * ((t >> 3) & 3) + (t & 3);
        if (lane < D / 8) {
            const int ks = lane >> 2, g = lane & 3;
            *reinterpret_cast<uint4*>(b + (((j * KS + ks) * 4 + g) * 16 + u) * 8) =
                *reinterpret_cast<const uint4*>(kn + 8 * lane);
        }
        const int kk = t >> 5, g = (t >> 3) & 3, e = t & 7;
        for (int d = lane; d < D; d += 64)
            b[64 * D + ((((d >> 4) * 2 + kk) * 4 + g) * 16 + (d & 15)) * 8 + e] = vn[d];
    }
};

// ------------------------------------------------------------------------------------------
// fp32 operands (v_mfma_f32_16x16x4_f32).  S^T sub-tile j: token 16j + lr in A rows, element i of the
// accumulator is token 16j + 4lg + i.  O^T k-step (j, i): A = Vt[16dt + lr][16j + 4lg + i],
// B = P[lr][16j + 4lg + i] = the lane's own accumulator element.
template <int D>
struct F32Ops {
    static constexpr int KS = D / 4;
    static constexpr int DT = D / 16;
    static constexpr int EB = 4;
    struct Frag {
        float k[4][KS];
        float v[DT][16];
    };
    struct QReg {
        float b[KS];
    };
    __device__ static int tokC(int j, int lg, int i) { return 16 * j + 4 * lg + i; }

    __device__ static void load_q(QReg& q, const float* qr, int n_heads, int lane) {
        const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) q.b[ks] = lr < n_heads ? qr[lr * D + 4 * ks + lg] : 0.f;
    }
    __device__ static void load(Frag& f, const char* base, int lane) {
        const int lr = lane & 15, lg = lane >> 4;
        const float* k = reinterpret_cast<const float*>(base);
        const float* vt = k + 64 * D;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) f.k[j][ks] = k[(16 * j + lr) * D + 4 * ks + lg];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj)
                f.v[dt][jj] = vt[(16 * dt + lr) * 64 + 16 * (jj >> 2) + 4 * lg + (jj & 3)];
    }
    __device__ static void pin_k(const Frag& f) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) asm volatile("" :: "v"(f.k[j][ks]) : "memory");
    }
    __device__ static float dot_q_new(const QReg& q, const float* kn, int lane) {
        const int lg = lane >> 4;
        float acc = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = fmaf(q.b[ks], kn[4 * ks + lg], acc);
        return acc;
    }
    __device__ static void load_vnew(const float* vn, int lane, float v[DT][4]) {
        const int lg = lane >> 4;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[dt][i] = vn[16 * dt + 4 * lg + i];
    }
    __device__ static void qk(const Frag& f, const QReg& q, f32x4 s[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(f.k[j][ks], q.b[ks], acc, 0, 0, 0);
            s[j] = acc;
        }
    }
    __device__ static void pv(const Frag& f, const float p[16], f32x4 o[DT]) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(f.v[dt][jj], p[jj], o[dt], 0, 0, 0);
    }
    __device__ static void write_current(char* base, int cur, const float* kn, const float* vn, int lane) {
        float* k = reinterpret_cast<float*>(base);
        float* vt = k + 64 * D;
        for (int d = lane; d < D; d += 64) {
            k[cur * D + d] = kn[d];
            vt[d * 64 + cur] = vn[d];
        }
    }
};

struct TileDesc {
    const char* base;
    unsigned long long mask;  // valid tokens of the tile
    bool cur;                 // the ring tile whose slot receives the current token
};

// ------------------------------------------------------------------------------------------
constexpr int kGroupsPerCU = 1;

template <typename Ops, typename T, int D>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(DecodeParams p) {
    constexpr int DT = D / 16;
    __shared__ float s_o[kWaves][kHeads][D + 4];  // rows padded: 16-byte stores of a wave hit all banks
    __shared__ float s_m[kWaves][kHeads];
    __shared__ float s_l[kWaves][kHeads];
    __shared__ int2 s_ent[kStage];
    __shared__ int s_next;
    __shared__ int s_ns[kMaxReq];
    __shared__ int s_pre[kMaxReq + 1];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int w = blockIdx.x;
    const bool dev_counts = p.n_sel_dev != nullptr;
    if (dev_counts) tile_split(p.n_sel_dev, p.n_sel, p.n_ring, p.row, p.n_req, s_ns, s_pre);
    // both sources are uniform: the LDS values are moved to scalar registers
    auto prefix = [&](int r) { return dev_counts ? __builtin_amdgcn_readfirstlane(s_pre[r]) : p.tile_prefix[r]; };
    const long long T_ = prefix(p.n_req), G = split_groups(p.n_groups, T_);
    if (dev_counts && w == 0 && (int)threadIdx.x < p.n_req) {
        // the groups whose tile ranges meet each request's tiles, for the merge (which would otherwise
        // repeat this split in every one of its groups before reading a partial)
        const int rr = threadIdx.x;
        p.mrange[2 * rr] = split_group_of(s_pre[rr], T_, G);
        p.mrange[2 * rr + 1] = split_group_of(s_pre[rr + 1] - 1, T_, G);
    }
    if (w >= G) return;
    const int a = (int)split_bound(w, T_, G);
    const int b = (int)split_bound(w + 1, T_, G);
    const size_t block_bytes = (size_t)2 * 64 * D * Ops::EB;

    int r = 0;
    while (r + 1 < p.n_req && prefix(r + 1) <= a) ++r;

    for (; r < p.n_req && prefix(r) < b; ++r) {
        const int P0 = prefix(r);
        const int lo = max(a, P0) - P0;
        const int hi = min(b, prefix(r + 1)) - P0;
        const int L = p.seq_len[r];
        const int ws = p.ws[r];
        const int n_sel = dev_counts ? __builtin_amdgcn_readfirstlane(s_ns[r]) : p.n_sel[r];
        const int2* tbl = p.table + p.tbl_off[r];
        const int row = p.row[r];
        char* ring_r = p.ring + (size_t)row * p.ring_req_bytes;
        const T* kn = p.k_new ? static_cast<const T*>(p.k_new) + (size_t)row * D : nullptr;
        const T* vn = p.v_new ? static_cast<const T*>(p.v_new) + (size_t)row * D : nullptr;
        const int cur_slot = (L - 1) % p.win_cap;
        const int cur_chunk = cur_slot >> 6;
        const int cur_row = cur_slot & 63;

        typename Ops::QReg q;
        const T* q_r = static_cast<const T*>(p.q) + (size_t)row * p.n_heads * D;
        Ops::load_q(q, q_r, p.n_heads, lane);

        float m_run = -INFINITY, l_run = 0.f;
        f32x4 o[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

        const char* cur_base = nullptr;
        // The segment's tiles go to the waves on demand: each wave takes the next tile from an LDS
        // counter when it finishes one, so waves the scheduler favours take more and all of them end
        // together.  The table entries of the segment's block tiles are staged in LDS, kStage at a time.
        for (int c0 = lo; c0 < hi; c0 += kStage) {
            const int c1 = min(hi, c0 + kStage);
            for (int e = threadIdx.x; e < c1 - c0; e += kThreads) {
                const int j = c0 + e;
                s_ent[e] = j < n_sel ? tbl[j] : make_int2(0, -1);
            }
            if (threadIdx.x == 0) s_next = c0;
            __syncthreads();
            auto desc = [&](int j) -> TileDesc {
                TileDesc d;
                d.cur = false;
                if (j < n_sel) {
                    const int2 ent = s_ent[j - c0];
                    const int blk = ent.x, slot = ent.y;
                    const int nv = min(64, max(0, ws - 64 * blk));
                    const bool ok = slot >= 0 && slot < p.n_slots && nv > 0;
                    d.mask = !ok ? 0ull : (nv >= 64 ? ~0ull : ((1ull << nv) - 1ull));
                    d.base = p.pool + (size_t)(ok ? slot : 0) * block_bytes;
                } else {
                    const int c = (p.ring_first[r] + (j - n_sel)) % p.n_chunks;
                    d.base = ring_r + (size_t)c * block_bytes;
                    const int s = 64 * c + lane;
                    int back = (L - 1 - s) % p.win_cap;
                    if (back < 0) back += p.win_cap;
                    const int pos = L - 1 - back;
                    d.mask = __ballot(pos >= ws);
                    if (kn && c == cur_chunk) {
                        // the slot still holds an old token: the current one is added after the loop
                        d.cur = true;
                        d.mask &= ~(1ull << cur_row);
                    }
                }
                return d;
            };
            auto compute = [&](typename Ops::Frag& f, const TileDesc& d) {
                f32x4 s[4];
                Ops::qk(f, q, s);
                float sv[16];
                float mx = -INFINITY;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = Ops::tokC(j, lg, i);
                        const float v = ((d.mask >> t) & 1ull) ? s[j][i] * p.scale_log2 : -INFINITY;
                        sv[4 * j + i] = v;
                        mx = fmaxf(mx, v);
                    }
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float m_new = fmaxf(m_run, mx);
                // a head with no valid token yet keeps (m, l, o) = (-inf, 0, 0)
                const float m_use = m_new == -INFINITY ? 0.f : m_new;
                const float corr = fast_exp2(m_run - m_use);
                float ps = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    sv[e] = fast_exp2(sv[e] - m_use);
                    ps += sv[e];
                }
                l_run = l_run * corr + ps;
                m_run = m_new;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
                Ops::pv(f, sv, o);
            };
            // One tile in registers per wave; latency is hidden by the other waves of the SIMD, which
            // stream their tiles while this one computes.  Every tile has a valid base and nothing but
            // the tile's own loads sits between them and the matrix products, so the products wait
            // only for the operands they read.
            for (;;) {
                int j = 0;
                if (lane == 0) j = atomicAdd(&s_next, 1);
                j = __builtin_amdgcn_readfirstlane(j);
                if (j >= c1) break;
                const TileDesc d = desc(j);
                if (d.cur) cur_base = d.base;
                // a tile with no valid token (a table entry inside the window, which device-side counts
                // include) is not read; the branch comes before any load of the tile
                if (d.mask == 0) continue;
                typename Ops::Frag f;
                Ops::load(f, d.base, lane);
                Ops::pin_k(f);
                compute(f, d);
            }
            __syncthreads();  // every wave is done with s_ent and s_next
        }

        // ---- the current token: folded into this wave's state, then appended to the ring ----
        if (cur_base) {
            float part = Ops::dot_q_new(q, kn, lane);
            part += __shfl_xor(part, 16, 64);
            part += __shfl_xor(part, 32, 64);
            const float s_cur = part * p.scale_log2;
            const float m_new = fmaxf(m_run, s_cur);
            const float corr = fast_exp2(m_run - m_new);
            const float pc = fast_exp2(s_cur - m_new);
            l_run = l_run * corr + (lg == 0 ? pc : 0.f);
            m_run = m_new;
            float vv[DT][4];
            Ops::load_vnew(vn, lane, vv);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) o[dt][i] = o[dt][i] * corr + pc * vv[dt][i];
            Ops::write_current(const_cast<char*>(cur_base), cur_row, kn, vn, lane);
        }

        // ---- combine the waves of this segment ----
        // the segment's maximum per head first; each wave then scales its own state to it, so the
        // final reduction is a plain sum over the waves
        float l_tot = l_run + __shfl_xor(l_run, 16, 64);
        l_tot += __shfl_xor(l_tot, 32, 64);
        if (lg == 0) s_m[wave][lr] = m_run;
        __syncthreads();
        float M = -INFINITY;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) M = fmaxf(M, s_m[v][lr]);
        const float sc = m_run == -INFINITY ? 0.f : fast_exp2(m_run - M);
        if (lg == 0) s_l[wave][lr] = sc * l_tot;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<float4*>(&s_o[wave][lr][16 * dt + 4 * lg]) =
                make_float4(sc * o[dt][0], sc * o[dt][1], sc * o[dt][2], sc * o[dt][3]);
        __syncthreads();
        const int pidx = w + r;
        for (int e = threadIdx.x; e < kHeads * D; e += kThreads) {
            const int h = e / D, d = e % D;
            float acc = 0.f;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) acc += s_o[v][h][d];
            p.part_o[((size_t)pidx * kHeads + h) * D + d] = acc;
            if (d == 0) {
                float Mh = -INFINITY, lsum = 0.f;
#pragma unroll
                for (int v = 0; v < kWaves; ++v) {
                    Mh = fmaxf(Mh, s_m[v][h]);
                    lsum += s_l[v][h];
                }
                p.part_ml[((size_t)pidx * kHeads + h) * 2 + 0] = Mh;
                p.part_ml[((size_t)pidx * kHeads + h) * 2 + 1] = lsum;
            }
        }
        __syncthreads();
    }
}

// One group per (request, head, 32 output columns).  Combines the partials of groups w_lo..w_hi
// (index w + r) in one pass: 16 partial subsets per column, each with a running maximum (4 partials
// loaded at once), then the subsets are rescaled to the common maximum in LDS.
constexpr int kMergeCols = 32;
constexpr int kMergeThreads = 512;
constexpr int kMergeSub = kMergeThreads / kMergeCols;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams p) {
    __shared__ float s_acc[kMergeSub][kMergeCols];
    __shared__ float s_l[kMergeSub][kMergeCols];
    __shared__ float s_m[kMergeSub][kMergeCols];
    constexpr int NC = D / kMergeCols;
    const int c = blockIdx.x % NC;
    const int rh = blockIdx.x / NC;
    const int r = rh / p.n_heads;
    const int h = rh % p.n_heads;
    const int col = threadIdx.x % kMergeCols;
    const int d = c * kMergeCols + col;
    const int sub = threadIdx.x / kMergeCols;
    // the groups whose tile ranges meet request r's tiles
    int w0 = p.w_lo[r], w1 = p.w_hi[r];
    if (p.n_sel_dev) {  // computed by the attention kernel from the same counts
        w0 = p.mrange[2 * r];
        w1 = p.mrange[2 * r + 1];
    }
    float m = -INFINITY, acc = 0.f, lsum = 0.f;
    for (int w = w0 + sub; w <= w1; w += 4 * kMergeSub) {
        float m4[4], o4[4], l4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int wu = min(w + u * kMergeSub, w1);  // clamped: the extra reads are discarded
            const size_t pi = (size_t)(wu + r) * kHeads + h;
            m4[u] = p.part_ml[pi * 2];
            l4[u] = p.part_ml[pi * 2 + 1];
            o4[u] = p.part_o[pi * D + d];
        }
        float mx = m;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (w + u * kMergeSub <= w1) mx = fmaxf(mx, m4[u]);
        if (mx != -INFINITY) {
            const float corr = fast_exp2(m - mx);  // m = -inf gives 0
            acc *= corr;
            lsum *= corr;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float sc = w + u * kMergeSub <= w1 ? fast_exp2(m4[u] - mx) : 0.f;
                acc += sc * o4[u];
                lsum += sc * l4[u];
            }
            m = mx;
        }
    }
    s_acc[sub][col] = acc;
    s_l[sub][col] = lsum;
    s_m[sub][col] = m;
    __syncthreads();
    if (sub == 0) {
        float M = -INFINITY;
#pragma unroll
        for (int s = 0; s < kMergeSub; ++s) M = fmaxf(M, s_m[s][col]);
        float a = 0.f, l = 0.f;
#pragma unroll
        for (int s = 0; s < kMergeSub; ++s) {
            const float ms = s_m[s][col];
            const float sc = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
            a += sc * s_acc[s][col];
            l += sc * s_l[s][col];
        }
        p.out[((size_t)p.row[r] * p.n_heads + h) * D + d] = a / l;
    }
}

struct DecodePlan {
    int G = 0;
    int total_tiles = 0;
    size_t part_o_off = 0, part_ml_off = 0, mrange_off = 0, total = 0;
};

lsa_status decode_check(const lsa_decode_args* a) {
    LSA_CHECK_ARG(a != nullptr, "lsa_sparse_decode: null args");
    LSA_CHECK_ARG(a->n_req >= 1 && a->n_req <= kMaxReq, "lsa_sparse_decode: n_req=%d outside 1..%d", a->n_req, kMaxReq);
    LSA_CHECK_SUP(dtype_ok(a->dtype), "lsa_sparse_decode: dtype %d", a->dtype);
    LSA_CHECK_SUP(a->head_dim == 64 || a->head_dim == 128, "lsa_sparse_decode: head_dim=%d (64 or 128)", a->head_dim);
    LSA_CHECK_SUP(a->n_heads >= 1 && a->n_heads <= kHeads, "lsa_sparse_decode: n_heads=%d (1..16)", a->n_heads);
    LSA_CHECK_ARG(a->win_cap >= 64 && a->win_cap % 64 == 0, "lsa_sparse_decode: win_cap=%d (multiple of 64)", a->win_cap);
    LSA_CHECK_ARG(a->reserved0 == 0 && a->reserved1 == 0, "lsa_sparse_decode: reserved fields must be 0");
    LSA_CHECK_ARG(a->max_groups >= 0, "lsa_sparse_decode: max_groups=%d", a->max_groups);
    LSA_CHECK_ARG(a->tbl_off && a->n_sel && a->seq_len && a->window, "lsa_sparse_decode: null host array");
    LSA_CHECK_ARG((a->k_new == nullptr) == (a->v_new == nullptr), "lsa_sparse_decode: give both k_new and v_new or neither");
    if (a->req_rows) {  // rows of distinct requests: each writes its own ring row and output row
        for (int r = 0; r < a->n_req; ++r) {
            LSA_CHECK_ARG(a->req_rows[r] >= 0, "lsa_sparse_decode: req_rows[%d]=%d", r, a->req_rows[r]);
            for (int r2 = 0; r2 < r; ++r2)
                LSA_CHECK_ARG(a->req_rows[r2] != a->req_rows[r], "lsa_sparse_decode: req_rows[%d] == req_rows[%d]", r2, r);
        }
    }
    LSA_CHECK_ARG(a->n_slots_total >= 0, "lsa_sparse_decode: n_slots_total=%d", a->n_slots_total);
    return LSA_OK;
}

lsa_status decode_plan(const lsa_decode_args* a, DecodePlan* P, bool sizing_only) {
    lsa_status st = decode_check(a);
    if (st != LSA_OK) return st;
    long long T = 0;
    if (!sizing_only) {
        const int n_chunks = a->win_cap / 64;
        for (int r = 0; r < a->n_req; ++r) {
            const int L = a->seq_len[r], W = a->window[r];
            LSA_CHECK_ARG(L >= 1, "lsa_sparse_decode: seq_len[%d]=%d", r, L);
            LSA_CHECK_ARG(W >= 1 && W <= a->win_cap, "lsa_sparse_decode: window[%d]=%d outside 1..win_cap", r, W);
            LSA_CHECK_ARG(a->n_sel[r] >= 0 && a->tbl_off[r] >= 0, "lsa_sparse_decode: n_sel/tbl_off[%d] negative", r);
            const int ws = std::max(0, L - W);
            const int ring = std::min(n_chunks, (L - 1) / 64 - ws / 64 + 1);
            T += (long long)a->n_sel[r] + ring;
        }
        LSA_CHECK_ARG(T < (1ll << 30), "lsa_sparse_decode: too many tiles");
    }
    DeviceInfo dev;
    st = current_device(&dev);
    if (st != LSA_OK) return st;
    const int g_all = dev.cu_count * kGroupsPerCU;
    const int g_max = a->max_groups > 0 ? std::min(a->max_groups, g_all) : g_all;
    P->total_tiles = (int)T;
    // with device-side counts the host knows only the capacities: every group is launched and the
    // kernels use min(G, T) of them
    P->G = sizing_only || a->n_sel_dev ? g_max
                                       : (int)std::max<long long>(1, std::min<long long>(g_max, (T + kWaves - 1) / kWaves));
    const int n_part = g_max + a->n_req;
    size_t off = 0;
    P->part_o_off = off;
    off = align_up(off + (size_t)n_part * kHeads * a->head_dim * sizeof(float), 256);
    P->part_ml_off = off;
    off = align_up(off + (size_t)n_part * kHeads * 2 * sizeof(float), 256);
    P->mrange_off = off;
    off = align_up(off + (size_t)a->n_req * 2 * sizeof(int), 256);
    P->total = off;
    return LSA_OK;
}

template <typename Ops, typename T, int D>
lsa_status launch_decode(const lsa_decode_args* a, const DecodePlan& P, char* ws, hipStream_t stream) {
    DecodeParams dp{};
    dp.q = a->q;
    dp.k_new = a->k_new;
    dp.v_new = a->v_new;
    dp.ring = static_cast<char*>(a->ring);
    const size_t bb = lsa_block_bytes(a->dtype, a->head_dim);
    dp.ring_req_bytes = (long long)(a->win_cap / 64) * (long long)bb;
    dp.pool = static_cast<const char*>(a->pool);
    dp.table = reinterpret_cast<const int2*>(a->table);
    dp.part_o = reinterpret_cast<float*>(ws + P.part_o_off);
    dp.part_ml = reinterpret_cast<float*>(ws + P.part_ml_off);
    dp.mrange = reinterpret_cast<int*>(ws + P.mrange_off);
    dp.n_req = a->n_req;
    dp.n_heads = a->n_heads;
    dp.n_chunks = a->win_cap / 64;
    dp.win_cap = a->win_cap;
    dp.n_slots = a->n_slots_total;
    dp.n_sel_dev = a->n_sel_dev;
    dp.n_groups = P.G;
    dp.scale_log2 = a->scale * 1.4426950408889634f;
    MergeParams mp{};
    for (int r = 0; r < a->n_req; ++r) {
        const int L = a->seq_len[r], W = a->window[r];
        const int wsr = std::max(0, L - W);
        const int ring = std::min(dp.n_chunks, (L - 1) / 64 - wsr / 64 + 1);
        dp.seq_len[r] = L;
        dp.ws[r] = wsr;
        dp.tbl_off[r] = a->tbl_off[r];
        dp.n_sel[r] = a->n_sel[r];
        dp.n_ring[r] = ring;
        dp.ring_first[r] = (wsr / 64) % dp.n_chunks;
        dp.row[r] = mp.row[r] = a->req_rows ? a->req_rows[r] : r;
        mp.n_sel[r] = a->n_sel[r];
        mp.n_ring[r] = ring;
    }
    if (!a->n_sel_dev) {
        int pre = 0;
        for (int r = 0; r < a->n_req; ++r) {
            dp.tile_prefix[r] = pre;
            pre += dp.n_sel[r] + dp.n_ring[r];
        }
        dp.tile_prefix[a->n_req] = pre;
        // groups whose tile range meets request r's tiles (P.G <= T here)
        const long long TT = pre, G = P.G;
        int wcur = 0;
        for (int r = 0; r < a->n_req; ++r) {
            const long long t0 = dp.tile_prefix[r], t1 = dp.tile_prefix[r + 1];  // t1 > t0 always
            while (split_bound(wcur + 1, TT, G) <= t0) ++wcur;  // group whose range holds t0
            int wend = wcur;
            while (split_bound(wend + 1, TT, G) < t1) ++wend;   // group whose range holds t1-1
            mp.w_lo[r] = wcur;
            mp.w_hi[r] = wend;
        }
    }
    mp.part_o = dp.part_o;
    mp.part_ml = dp.part_ml;
    mp.mrange = dp.mrange;
    mp.out = a->out;
    mp.n_sel_dev = a->n_sel_dev;
    mp.n_req = a->n_req;
    mp.n_heads = a->n_heads;
    mp.n_groups = P.G;

    if (a->ev_attn_begin && a->ev_attn_end) {
        // the events take the dispatch's own start and end timestamps: no extra packets on the stream
        hipExtLaunchKernelGGL((attn_kernel<Ops, T, D>), dim3(P.G), dim3(kThreads), 0, stream, a->ev_attn_begin,
                              a->ev_attn_end, 0, dp);
    } else {
        hipLaunchKernelGGL((attn_kernel<Ops, T, D>), dim3(P.G), dim3(kThreads), 0, stream, dp);
    }
    LSA_HIP(hipGetLastError());
    hipLaunchKernelGGL((merge_kernel<D>), dim3(a->n_req * a->n_heads * (D / kMergeCols)), dim3(kMergeThreads), 0, stream, mp);
    LSA_HIP(hipGetLastError());
    return LSA_OK;
}

// ---- split-K partials without a workspace ------------------------------------------------------
// lsa_sparse_decode_noalloc keeps the partials in this array instead of a caller's workspace: one
// copy per device, held until the process ends, sized for kScratchGroups work-groups and the most
// requests of a call at head_dim 128.  Nothing in it needs to start at zero (every partial the
// merge reads is written by the same call's attention kernel); calls that overlap on one device
// share it and race.
constexpr int kScratchGroups = 320;
constexpr size_t kScratchBytes =
    (size_t)(kScratchGroups + kMaxReq) * kHeads * 128 * sizeof(float) +  // partial outputs (a 256 multiple)
    (size_t)(kScratchGroups + kMaxReq) * kHeads * 2 * sizeof(float) +    // (m, l) pairs (a 256 multiple)
    (size_t)kMaxReq * 2 * sizeof(int);                                   // the merge's group ranges
static __device__ __align__(256) char scratch[kScratchBytes];

// Device address of `scratch` on the current device: looked up once per device (each device holds
// its own copy of the array at its own address), never the host-side name of the array.
lsa_status scratch_address(char** out) {
    static std::mutex mu;
    static std::vector<char*> addr;
    int dev = -1;
    LSA_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lock(mu);
    if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        LSA_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (p == nullptr) return fail(LSA_ERR_HIP, "lsa_sparse_decode_noalloc: no device address for the scratch array");
        addr[dev] = static_cast<char*>(p);
    }
    *out = addr[dev];
    return LSA_OK;
}

// Checks shared by both entry points (everything but the workspace), then the plan.
lsa_status decode_prepare(const lsa_decode_args* a, DecodePlan* P) {
    lsa_status st = decode_check(a);
    if (st != LSA_OK) return st;
    LSA_CHECK_ARG(a->q && a->ring && a->out, "lsa_sparse_decode: null device pointer");
    bool any_sel = false;
    for (int r = 0; r < a->n_req; ++r) any_sel |= a->n_sel[r] > 0;
    LSA_CHECK_ARG(!any_sel || (a->pool && a->table && a->n_slots_total > 0),
                  "lsa_sparse_decode: selected blocks but no pool/table");
    st = decode_plan(a, P, false);
    if (st != LSA_OK) return st;
    LSA_CHECK_ARG(((uintptr_t)a->q % 16) == 0 && ((uintptr_t)a->ring % 16) == 0 &&
                      (a->pool == nullptr || ((uintptr_t)a->pool % 16) == 0) &&
                      (a->k_new == nullptr || ((uintptr_t)a->k_new % 16) == 0) &&
                      (a->table == nullptr || ((uintptr_t)a->table % 8) == 0),
                  "lsa_sparse_decode: q, ring, pool, k_new must be 16-byte aligned, table 8-byte aligned");
    return LSA_OK;
}

lsa_status decode_dispatch(const lsa_decode_args* a, const DecodePlan& P, char* ws, hipStream_t stream) {
    if (a->dtype == LSA_BF16) {
        if (a->head_dim == 128) return launch_decode<Bf16Ops<128>, uint16_t, 128>(a, P, ws, stream);
        return launch_decode<Bf16Ops<64>, uint16_t, 64>(a, P, ws, stream);
    }
    if (a->head_dim == 128) return launch_decode<F32Ops<128>, float, 128>(a, P, ws, stream);
    return launch_decode<F32Ops<64>, float, 64>(a, P, ws, stream);
}

}  // namespace
}  // namespace lsa

using namespace lsa;

extern "C" lsa_status lsa_sparse_decode_workspace(const lsa_decode_args* a, size_t* bytes) {
    DecodePlan P;
    lsa_status st = decode_plan(a, &P, true);
    if (st != LSA_OK) return st;
    LSA_CHECK_ARG(bytes != nullptr, "lsa_sparse_decode_workspace: bytes is null");
    *bytes = P.total;
    return LSA_OK;
}

extern "C" lsa_status lsa_sparse_decode(const lsa_decode_args* a, hipStream_t stream) {
    DecodePlan P;
    lsa_status st = decode_prepare(a, &P);
    if (st != LSA_OK) return st;
    if (a->workspace == nullptr || a->workspace_bytes < P.total)
        return fail(LSA_ERR_WORKSPACE, "lsa_sparse_decode: workspace of %zu bytes, need %zu",
                    a->workspace ? a->workspace_bytes : (size_t)0, P.total);
    return decode_dispatch(a, P, static_cast<char*>(a->workspace), stream);
}

extern "C" lsa_status lsa_sparse_decode_noalloc(const lsa_decode_args* a, hipStream_t stream) {
    DecodePlan P;
    lsa_status st = decode_prepare(a, &P);
    if (st != LSA_OK) return st;
    if (P.total > kScratchBytes)
        return fail(LSA_ERR_WORKSPACE,
                    "lsa_sparse_decode_noalloc: the call needs %zu bytes of partials, the static array holds "
                    "%zu (at most %d work-groups)", P.total, kScratchBytes, kScratchGroups);
    char* ws = nullptr;
    st = scratch_address(&ws);
    if (st != LSA_OK) return st;
    return decode_dispatch(a, P, ws, stream);
}
