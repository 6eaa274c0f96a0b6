// Host-side pieces of the LSA library: error reporting, device facts, struct sizes and the
// block-format packer.
#include <algorithm>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

#include "lsa_internal.hpp"

namespace lsa {

static thread_local std::string g_last_error;

lsa_status fail(lsa_status st, const char* fmt, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

lsa_status hip_fail(hipError_t e, const char* what) {
    return fail(LSA_ERR_HIP, "%s failed: %s (%d)", what, hipGetErrorString(e), (int)e);
}

lsa_status current_device(DeviceInfo* out) {
    static std::mutex mu;
    static std::vector<DeviceInfo> cache;
    int dev = -1;
    LSA_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lock(mu);
    if ((int)cache.size() <= dev) cache.resize(dev + 1);
    if (cache[dev].device < 0) {
        int cus = 0;
        LSA_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
        if (cus <= 0) return fail(LSA_ERR_HIP, "device %d reports %d compute units", dev, cus);
        cache[dev].device = dev;
        cache[dev].cu_count = cus;
    }
    *out = cache[dev];
    return LSA_OK;
}

}  // namespace lsa

using namespace lsa;

extern "C" {

const char* lsa_last_error(void) { return g_last_error.c_str(); }

int32_t lsa_abi_version(void) { return LSA_ABI_VERSION; }

size_t lsa_struct_size(int32_t which) {
    switch (which) {
        case 0: return sizeof(lsa_refresh_args);
        case 1: return sizeof(lsa_gather_args);
        case 2: return sizeof(lsa_decode_args);
        case 3: return sizeof(lsa_latent_args);
        case 4: return sizeof(lsa_denoise_args);
        case 5: return sizeof(lsa_device_gather_args);
        default: return 0;
    }
}

size_t lsa_block_bytes(int32_t dtype, int32_t head_dim) {
    if (!dtype_ok(dtype) || (head_dim != 64 && head_dim != 128)) return 0;
    return (size_t)2 * LSA_BLOCK_TOKENS * head_dim * elem_bytes(dtype);
}

}  // extern "C"

namespace {

// Element offsets inside a bf16 block (matrix-core fragment order: every 1 KiB run is one wave's
// 16-byte-per-lane operand load).
inline size_t bf16_key_off(int D, int t, int d) {
    const int KS = D / 32;
    const int j = 2 * (t >> 5) + ((t >> 2) & 1), u = 4 * ((t >> 3) & 3) + (t & 3);
    const int ks = d >> 5, g = (d >> 3) & 3, e = d & 7;
    return ((((size_t)j * KS + ks) * 4 + g) * 16 + u) * 8 + e;
}
inline size_t bf16_value_off(int D, int t, int d) {
    const int c = d >> 4, u = d & 15;
    const int kk = t >> 5, g = (t >> 3) & 3, e = t & 7;
    return (size_t)64 * D + ((((size_t)c * 2 + kk) * 4 + g) * 16 + u) * 8 + e;
}

}  // namespace

extern "C" {

lsa_status lsa_pack_blocks(int32_t dtype, int32_t head_dim, const void* k_tok, const void* v_tok,
                           int64_t pos0, int64_t n_tokens, void* dst, int64_t n_dst_blocks,
                           int32_t n_threads) {
    const size_t bb = lsa_block_bytes(dtype, head_dim);
    LSA_CHECK_SUP(bb != 0, "lsa_pack_blocks: dtype %d / head_dim %d not supported", dtype, head_dim);
    LSA_CHECK_ARG(pos0 >= 0 && n_tokens >= 0, "lsa_pack_blocks: pos0=%lld n_tokens=%lld",
                  (long long)pos0, (long long)n_tokens);
    LSA_CHECK_ARG(n_dst_blocks >= 1, "lsa_pack_blocks: n_dst_blocks=%lld", (long long)n_dst_blocks);
    if (n_tokens == 0) return LSA_OK;
    LSA_CHECK_ARG(k_tok && v_tok && dst, "lsa_pack_blocks: null pointer");
    LSA_CHECK_ARG(n_tokens <= n_dst_blocks * LSA_BLOCK_TOKENS,
                  "lsa_pack_blocks: %lld tokens do not fit %lld blocks without overwriting",
                  (long long)n_tokens, (long long)n_dst_blocks);
    const int D = head_dim;
    const size_t eb = elem_bytes(dtype);
    const size_t row_bytes = (size_t)D * eb;
    const char* k = static_cast<const char*>(k_tok);
    const char* v = static_cast<const char*>(v_tok);
    char* out = static_cast<char*>(dst);

    // Work unit: the tokens of one 64-aligned position range (one destination block).
    const int64_t first_blk = pos0 / LSA_BLOCK_TOKENS;
    const int64_t last_blk = (pos0 + n_tokens - 1) / LSA_BLOCK_TOKENS;
    const int64_t n_units = last_blk - first_blk + 1;
    auto work = [&](int64_t u0, int64_t u1) {
        for (int64_t u = u0; u < u1; ++u) {
            const int64_t pb = first_blk + u;
            const int64_t p_lo = std::max<int64_t>(pos0, pb * LSA_BLOCK_TOKENS);
            const int64_t p_hi = std::min<int64_t>(pos0 + n_tokens, (pb + 1) * LSA_BLOCK_TOKENS);
            char* blk = out + (size_t)(pb % n_dst_blocks) * bb;
            if (dtype == LSA_BF16) {
                uint16_t* b16 = reinterpret_cast<uint16_t*>(blk);
                for (int64_t p = p_lo; p < p_hi; ++p) {
                    const int t = (int)(p % LSA_BLOCK_TOKENS);
                    const uint16_t* kr = reinterpret_cast<const uint16_t*>(k + (size_t)(p - pos0) * row_bytes);
                    const uint16_t* vr = reinterpret_cast<const uint16_t*>(v + (size_t)(p - pos0) * row_bytes);
                    for (int d = 0; d < D; d += 8) std::memcpy(b16 + bf16_key_off(D, t, d), kr + d, 16);
                    for (int d = 0; d < D; ++d) b16[bf16_value_off(D, t, d)] = vr[d];
                }
                continue;
            }
            char* vt = blk + (size_t)LSA_BLOCK_TOKENS * row_bytes;
            for (int64_t p = p_lo; p < p_hi; ++p) {
                const int row = (int)(p % LSA_BLOCK_TOKENS);
                const size_t src = (size_t)(p - pos0) * row_bytes;
                std::memcpy(blk + row * row_bytes, k + src, row_bytes);
            }
            for (int d = 0; d < D; ++d) {
                char* dcol = vt + (size_t)d * LSA_BLOCK_TOKENS * eb;
                for (int64_t p = p_lo; p < p_hi; ++p) {
                    const int row = (int)(p % LSA_BLOCK_TOKENS);
                    std::memcpy(dcol + row * eb, v + (size_t)(p - pos0) * row_bytes + d * eb, eb);
                }
            }
        }
    };
    int nt = n_threads > 0 ? n_threads : (int)std::min<unsigned>(16, std::max(1u, std::thread::hardware_concurrency()));
    nt = (int)std::min<int64_t>(nt, std::max<int64_t>(1, n_units / 64));
    if (nt <= 1) {
        work(0, n_units);
        return LSA_OK;
    }
    std::vector<std::thread> th;
    th.reserve(nt);
    for (int t = 0; t < nt; ++t) {
        const int64_t u0 = n_units * t / nt, u1 = n_units * (t + 1) / nt;
        th.emplace_back(work, u0, u1);
    }
    for (auto& x : th) x.join();
    return LSA_OK;
}

}  // extern "C"
