// Host-side run of libwc's encoder and planner under AddressSanitizer and
// UndefinedBehaviorSanitizer (built and run by tests/test_host_sanitizers.py,
// with kernel_stubs.cpp standing in for the GPU side).
//
// For seeded inputs and every container option the GPU decoder takes, it
// writes a container, plans it, and calls each decode entry point with the
// container itself as the "device" copy: the stand-in launches check that
// every pointer they are handed lies inside it.  Then it plans thousands of
// corrupted copies (bit flips and byte overwrites in the header and metadata,
// truncations): wc_plan must return a status without reading outside the
// buffer, and a plan it accepts must again only hand in-bounds parameters to
// the launches.  Invalid options must be refused by the encoder.  Exit status
// 0 and the line "host_fuzz ok" mean every check passed; a sanitizer report
// aborts the run.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/wc.h"
#include "stub_state.h"

namespace {

struct Rng {   // splitmix64
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    uint32_t below(uint32_t n) { return (uint32_t)(next() % n); }
};

int failures = 0;
#define EXPECT(cond, ...)                                  \
    do {                                                   \
        if (!(cond)) {                                     \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);             \
            std::fprintf(stderr, "\n");                    \
            ++failures;                                    \
        }                                                  \
    } while (0)

// bf16 bit patterns with the shape of trained weights: a narrow exponent
// range, random signs and mantissas, a sprinkle of special values
std::vector<uint16_t> weights(Rng& r, uint64_t n, int kind) {
    std::vector<uint16_t> w(n);
    for (auto& v : w) {
        const uint64_t x = r.next();
        if (kind == 0) {
            v = (uint16_t)x;
        } else if (kind == 1) {
            v = 0x3F80;
        } else {
            const uint32_t e = 117 + (uint32_t)(x % 9) - (uint32_t)((x >> 8) % 3 == 0 ? 4 : 0);
            v = (uint16_t)(((x >> 20) & 1) << 15 | e << 7 | ((x >> 32) & 0x7F));
            if (kind == 3 && (x >> 40) % 97 == 0) v = (uint16_t)((x >> 48) % 2 ? 0x7F80 : 0x0001);
        }
    }
    return w;
}

std::vector<uint8_t> codes(Rng& r, uint64_t n, int spread) {
    std::vector<uint8_t> c(n);
    for (auto& v : c) {
        int s = 0;
        for (int k = 0; k < 4; ++k) s += (int)(r.next() % (2 * spread + 1)) - spread;
        v = (uint8_t)(128 + s);
    }
    return c;
}

uint8_t* aligned_copy(const uint8_t* b, uint64_t n) {
    uint8_t* p = static_cast<uint8_t*>(std::aligned_alloc(256, (n + 255) / 256 * 256 + 256));
    std::memcpy(p, b, n);
    return p;
}

// Plan a container and run every entry point that applies to it; returns the
// plan status.  A plan that is accepted must hand in-bounds parameters to
// every launch (the stand-ins abort otherwise).
int plan_and_decode(const uint8_t* blob, uint64_t bytes, bool expect_ok) {
    wc_plan_t* plan = nullptr;
    const int st = wc_plan(blob, bytes, 0, &plan);
    if (expect_ok) EXPECT(st == WC_OK, "wc_plan of a container just written: %d", st);
    if (st != WC_OK) {
        EXPECT(plan == nullptr || st == WC_OK, "a failed wc_plan left a plan");
        return st;
    }
    uint64_t n = 0, cb = 0, sb = 0, ng = 0;
    uint32_t nt = 0, kc = 0, kd = 0, grid = 0, lds = 0, ver = 0, kind = 0, coder = 0;
    EXPECT(wc_plan_info(plan, &n, &nt, nullptr, nullptr) == WC_OK, "wc_plan_info");
    std::vector<uint64_t> offs(nt + 1), nums(nt + 1);
    EXPECT(wc_plan_info(plan, nullptr, nullptr, offs.data(), nums.data()) == WC_OK, "wc_plan_info tables");
    EXPECT(wc_plan_stats(plan, &cb, &sb, &ng, &kc, &kd, &grid, &lds) == WC_OK, "wc_plan_stats");
    EXPECT(wc_plan_format(plan, &ver, &kind, &coder) == WC_OK, "wc_plan_format");
    EXPECT(cb <= bytes, "container_bytes %llu beyond the %llu given", (unsigned long long)cb,
           (unsigned long long)bytes);
    uint64_t sum = 0;
    for (uint32_t t = 0; t < nt; ++t) {
        EXPECT(offs[t] == sum, "tensor %u offset", t);
        sum += nums[t];
    }
    EXPECT(sum == n, "tensor numels sum");

    g_stub.lo = blob;
    g_stub.hi = blob + bytes;
    std::vector<uint8_t> out(2 * n + 16);
    uint8_t* out_al = out.data() + ((16 - (reinterpret_cast<uintptr_t>(out.data()) & 15u)) & 15u);
    const uint64_t before = g_stub.launches;
    if (kind == 0) {
        EXPECT(wc_decode_async(plan, blob, reinterpret_cast<uint16_t*>(out_al), nullptr) == WC_OK, "decode");
        EXPECT(wc_decode_u8_async(plan, blob, out_al, nullptr) == WC_ERR_INVALID_ARG, "u8 entry on bf16");
        EXPECT(n == 0 || g_stub.launches == before + 1, "one decode launch");
        // the fused product over the tensors whose numel has a row length
        // of a multiple of 8 that is at least 4096 (group_max_elems)
        std::vector<wc_gemv_operand> ops;
        std::vector<std::vector<uint16_t>> xs;
        std::vector<std::vector<float>> ys;
        for (uint32_t t = 0; t < nt && ops.size() < 16; ++t) {
            uint32_t cols = 0;
            for (uint32_t c = 4096; c <= 16384 && !cols; c += 8)
                if (nums[t] && nums[t] % c == 0) cols = c;
            if (!cols || nums[t] >= (1ull << 32)) break;
            xs.emplace_back(cols + 8);
            ys.emplace_back(nums[t] / cols);
            uint16_t* xa = xs.back().data() + ((16 - (reinterpret_cast<uintptr_t>(xs.back().data()) & 15u)) & 15u) / 2;
            ops.push_back({t, cols, xa, ys.back().data()});
        }
        if (!ops.empty() && ops[0].tensor == 0) {
            uint64_t wb = 0;
            const int s1 = wc_decode_gemv_work_bytes(plan, ops.data(), (uint32_t)ops.size(), &wb);
            if (s1 == WC_OK) {
                void* work = std::aligned_alloc(256, (wb + 255) / 256 * 256 + 256);
                EXPECT(wc_decode_gemv_async(plan, blob, ops.data(), (uint32_t)ops.size(), work, wb, nullptr) ==
                           WC_OK,
                       "decode_gemv");
                EXPECT(wc_decode_gemv_async(plan, blob, ops.data(), (uint32_t)ops.size(), work, wb ? wb - 1 : 0,
                                            nullptr) != WC_OK || wb == 0,
                       "decode_gemv with a short work buffer");
                std::free(work);
            }
        }
    } else {
        EXPECT(wc_decode_u8_async(plan, blob, out_al, nullptr) == WC_OK, "decode_u8");
        EXPECT(wc_decode_async(plan, blob, reinterpret_cast<uint16_t*>(out_al), nullptr) == WC_ERR_INVALID_ARG,
               "bf16 entry on u8");
    }
    // the debug status word: present (and clear) only when the plan was made
    // with WC_DEBUG=1, and handed to the launches
    {
        const char* dbg = std::getenv("WC_DEBUG");
        const bool debug = dbg && std::strcmp(dbg, "1") == 0;
        uint32_t word = 7;
        const int ds = wc_plan_debug_status(plan, &word, 1);
        EXPECT(ds == (debug ? WC_OK : WC_ERR_INVALID_ARG), "wc_plan_debug_status with WC_DEBUG=%d: %d", debug, ds);
        if (debug) EXPECT(word == 0, "a fresh debug status word reads %u", word);
        EXPECT(n == 0 || (g_stub.last_status != nullptr) == debug, "the launches' status pointer");
        EXPECT(wc_plan_debug_status(plan, nullptr, 0) == WC_ERR_INVALID_ARG, "null status");
    }
    // misaligned and null device pointers are refused
    if (n) {
        EXPECT(wc_decode_async(plan, blob + 1, reinterpret_cast<uint16_t*>(out_al), nullptr) == WC_ERR_INVALID_ARG,
               "misaligned blob");
        EXPECT(wc_decode_async(plan, nullptr, reinterpret_cast<uint16_t*>(out_al), nullptr) == WC_ERR_INVALID_ARG,
               "null blob");
    }
    g_stub.lo = g_stub.hi = nullptr;
    wc_plan_destroy(plan);
    return st;
}

// Corrupt copies of a container: every one is planned (and decoded when
// accepted) under the sanitizers.
void corrupt(Rng& r, const uint8_t* blob, uint64_t bytes, uint64_t meta_end, int rounds) {
    for (int i = 0; i < rounds; ++i) {
        uint8_t* b = aligned_copy(blob, bytes);
        uint64_t len = bytes;
        const uint32_t kind = r.below(4);
        const uint64_t span = meta_end ? meta_end : bytes;
        if (kind == 0) {                       // one bit in the header or metadata
            const uint64_t k = r.next() % span;
            b[k] ^= (uint8_t)(1u << r.below(8));
        } else if (kind == 1) {                // a byte overwritten anywhere
            b[r.next() % bytes] = (uint8_t)r.next();
        } else if (kind == 2) {                // a 64-bit field set to an extreme
            const uint64_t k = (r.next() % (span / 8)) * 8;
            const uint64_t v = r.below(2) ? ~0ull : (1ull << r.below(64));
            std::memcpy(b + k, &v, 8);
        } else {                               // truncated
            len = r.next() % bytes;
        }
        plan_and_decode(b, len, false);
        std::free(b);
    }
}

uint64_t metadata_end(const uint8_t* blob, uint64_t bytes) {
    // the header, code lengths, tensor table, group table and gaps or lane
    // offsets come before the stream section, whose offset is at byte 88
    uint64_t v = 0;
    if (bytes >= 96) std::memcpy(&v, blob + 88, 8);
    return v >= 8 && v <= bytes ? v : bytes;
}

}  // namespace

int main(int argc, char** argv) {
    const int rounds = argc > 1 ? std::atoi(argv[1]) : 200;
    Rng r{20261203};
    const uint64_t sizes[] = {0, 1, 7, 8, 9, 4095, 4096, 4097, 20000, 70001};
    int containers = 0;
    for (int layout = 0; layout < 2; ++layout) {
        for (int coder = 0; coder < 2; ++coder) {
            if (layout == 1 && coder == 1) continue;     // rANS: lanes only
            for (int kind = 0; kind < 2; ++kind) {
                if (kind == 1 && layout == 1) continue;  // code planes: lanes only
                for (uint64_t n : sizes) {
                    wc_encode_opts o;
                    std::memset(&o, 0, sizeof(o));
                    o.layout = layout ? WC_LAYOUT_CHUNKS : WC_LAYOUT_LANES;
                    o.coder = coder ? WC_CODER_RANS : WC_CODER_HUFFMAN;
                    o.n_threads = 1 + r.below(3);
                    const uint32_t aligns[] = {8, 64, 120, 128};
                    o.group_align = aligns[r.below(4)];
                    o.group_max_elems = o.group_align * (1 + r.below(4096 / o.group_align));
                    if (layout == 1) {
                        o.chunks_per_group = r.below(2) ? 128 : 1000;
                        o.gap_bits = r.below(2) ? 5 : 8;
                    }
                    // split n into up to three tensors
                    const uint64_t a = n ? r.next() % (n + 1) : 0, b = a + (n - a ? r.next() % (n - a + 1) : 0);
                    const uint64_t numels[3] = {a, b - a, n - b};
                    uint8_t* blob = nullptr;
                    uint64_t bytes = 0;
                    int st;
                    if (kind == 0) {
                        const auto w = weights(r, n, (int)(n % 4));
                        const uint16_t* ts[3] = {w.data(), w.data() + a, w.data() + b};
                        st = wc_encode_host(ts, numels, 3, &o, &blob, &bytes);
                    } else {
                        const auto c = codes(r, n, 1 + (int)(n % 7));
                        const uint8_t* ts[3] = {c.data(), c.data() + a, c.data() + b};
                        st = wc_encode_u8_host(ts, numels, 3, &o, &blob, &bytes);
                    }
                    EXPECT(st == WC_OK, "encode layout=%d coder=%d kind=%d n=%llu A=%u M=%u: %d", layout, coder,
                           kind, (unsigned long long)n, o.group_align, o.group_max_elems, st);
                    if (st != WC_OK) continue;
                    ++containers;
                    setenv("WC_DEBUG", n % 2 ? "1" : "0", 1);   // debug plans for the odd sizes
                    plan_and_decode(blob, bytes, true);
                    corrupt(r, blob, bytes, metadata_end(blob, bytes), rounds);
                    unsetenv("WC_DEBUG");
                    wc_free_host(blob);
                }
            }
        }
    }
    // one-symbol codes are incomplete ("0" only): the planner must keep the
    // long-code lookup (which always advances) in the decode loops
    for (int kind = 0; kind < 2; ++kind) {
        const uint64_t n = 5000;
        const uint64_t numels[1] = {n};
        uint8_t* blob = nullptr;
        uint64_t bytes = 0;
        int st;
        if (kind == 0) {
            const std::vector<uint16_t> w(n, 0x3F80);
            const uint16_t* ts[1] = {w.data()};
            st = wc_encode_host(ts, numels, 1, nullptr, &blob, &bytes);
        } else {
            const std::vector<uint8_t> c(n, 77);
            const uint8_t* ts[1] = {c.data()};
            st = wc_encode_u8_host(ts, numels, 1, nullptr, &blob, &bytes);
        }
        EXPECT(st == WC_OK, "one-symbol encode kind %d: %d", kind, st);
        if (st != WC_OK) continue;
        plan_and_decode(blob, bytes, true);
        EXPECT(g_stub.last_no_long == 0, "one-symbol kind %d planned without the long-code lookup", kind);
        wc_free_host(blob);
    }
    // blocks of matrices (row lengths 4096 and 8192) for the fused product,
    // in every bf16 layout and coder
    for (int v = 0; v < 4; ++v) {
        wc_encode_opts o;
        std::memset(&o, 0, sizeof(o));
        o.layout = v >= 2 ? WC_LAYOUT_CHUNKS : WC_LAYOUT_LANES;
        o.coder = v == 1 ? WC_CODER_RANS : WC_CODER_HUFFMAN;
        o.gap_bits = v == 3 ? 5 : 0;
        o.chunks_per_group = v == 3 ? 300 : 0;
        const uint64_t numels[3] = {4096 * 5, 8192 * 3, 4096 * 2};
        const auto w = weights(r, numels[0] + numels[1] + numels[2], 2);
        const uint16_t* ts[3] = {w.data(), w.data() + numels[0], w.data() + numels[0] + numels[1]};
        uint8_t* blob = nullptr;
        uint64_t bytes = 0;
        const int st = wc_encode_host(ts, numels, 3, &o, &blob, &bytes);
        EXPECT(st == WC_OK, "encode matrices variant %d: %d", v, st);
        if (st != WC_OK) continue;
        ++containers;
        const uint64_t dots = g_stub.dot_launches;
        plan_and_decode(blob, bytes, true);
        EXPECT(g_stub.dot_launches == dots + 1, "variant %d: one fused launch", v);
        corrupt(r, blob, bytes, metadata_end(blob, bytes), rounds);
        wc_free_host(blob);
    }
    // options the encoder must refuse
    {
        const auto w = weights(r, 1000, 2);
        const uint16_t* ts[1] = {w.data()};
        const uint64_t numels[1] = {1000};
        struct Bad {
            uint32_t layout, coder, align, max_elems, seg, gap, max_len;
        } bad[] = {
            {0, 0, 12, 48, 0, 0, 0},     {0, 0, 4, 4096, 0, 0, 0},       {0, 0, 8, 8192, 0, 0, 0},
            {0, 0, 0, 0, 15873, 0, 0},   {0, 0, 0, 0, 65535, 0, 0},      {0, 1, 0, 0, 2047, 0, 0},
            {1, 1, 0, 0, 0, 0, 0},       {1, 0, 0, 0, 0, 6, 0},          {0, 0, 0, 0, 0, 5, 0},
            {0, 0, 0, 0, 0, 0, 25},      {0, 0, 128, 100, 0, 0, 0},      {0, 0, 64, 4096, 1000, 0, 0},
        };
        for (const Bad& x : bad) {
            wc_encode_opts o;
            std::memset(&o, 0, sizeof(o));
            o.layout = x.layout;
            o.coder = x.coder;
            o.group_align = x.align;
            o.group_max_elems = x.max_elems;
            o.seg_max_bits = x.seg;
            o.gap_bits = x.gap;
            o.max_code_len = x.max_len;
            uint8_t* blob = nullptr;
            uint64_t bytes = 0;
            const int st = wc_encode_host(ts, numels, 1, &o, &blob, &bytes);
            EXPECT(st == WC_ERR_INVALID_ARG, "bad options %u/%u/%u/%u/%u/%u/%u accepted: %d", x.layout, x.coder,
                   x.align, x.max_elems, x.seg, x.gap, x.max_len, st);
            wc_free_host(blob);
        }
        uint8_t* blob = nullptr;
        uint64_t bytes = 0;
        EXPECT(wc_encode_host(nullptr, numels, 1, nullptr, &blob, &bytes) == WC_ERR_INVALID_ARG, "null tensors");
        EXPECT(wc_plan(nullptr, 100, 0, nullptr) == WC_ERR_INVALID_ARG, "null plan arguments");
    }
    EXPECT(g_stub.live_allocs == 0, "%lld device allocations left", (long long)g_stub.live_allocs);
    std::printf("host_fuzz: %d containers, %d corrupt copies each, %llu launches checked (%llu fused), %d failures\n",
                containers, rounds, (unsigned long long)g_stub.launches, (unsigned long long)g_stub.dot_launches,
                failures);
    if (failures) return 1;
    std::printf("host_fuzz ok\n");
    return 0;
}
