// abi_fuzz.cpp -- random calls of every libnmspmv entry point with fake device
// addresses (never dereferenced: the kernel side is launch_stub.cpp, which
// checks the launch preconditions).  Shapes mix small valid ones, near-misses
// (K not a multiple of 8, N >= M, B = 33, ...) and the extremes of the 64-bit
// arguments; pointers are NULL, misaligned, or placed in one small address
// window so that buffers often overlap.  Built with
// -fsanitize=address,undefined by the CPU tests: undefined behaviour in the
// checks aborts the run, and so does a call that reaches the stub with
// arguments its rules should have rejected.  Each entry point must be seen
// both rejected (bad shape, bad argument) and accepted.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "nmspmv.h"

extern "C" long nmtest_launches(void);

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;

uint64_t next()   // splitmix64
{
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

uint64_t below(uint64_t n) { return next() % n; }

int64_t pick_rows()
{
    static const int64_t odd[] = {-1, -8, 0, (int64_t(1) << 31) - 1025, (int64_t(1) << 31) - 1024, int64_t(1) << 31,
                                  (int64_t(1) << 30) - 512, (int64_t(1) << 30) + 1, INT64_MAX, INT64_MIN};
    return below(5) ? (int64_t)below(40) : odd[below(sizeof odd / sizeof *odd)];
}

int64_t pick_k()
{
    static const int64_t odd[] = {0, 4, 12, 20, -8, -16, INT32_MAX, int64_t(INT32_MAX) - 7, int64_t(1) << 31,
                                  65536, 65544, INT64_MAX, INT64_MIN};
    return below(5) ? 8 * (int64_t)below(40) : odd[below(sizeof odd / sizeof *odd)];
}

int pick_b() { return below(6) ? 1 + (int)below(32) : (int)below(3) * 33 - 1; }   // else -1, 32, 65
int pick_dtype() { return below(10) ? (int)below(2) : 2 + (int)below(3) - 5 * (int)below(2); }
int pick_m() { return below(8) ? (below(2) ? 4 : 8) : (int)below(17); }
int pick_n(int M) { return below(8) ? 1 + (int)below(M > 1 ? M - 1 : 1) : (int)below(10); }

// An address in a 64 KB window (buffers there overlap often), NULL, or far apart.
void* pick_ptr(uintptr_t align)
{
    const uint64_t r = below(20);
    if (r == 0)
        return nullptr;
    uintptr_t base = r < 12 ? 0x100000 : 0x100000 + ((uintptr_t)below(1024) << 24);
    uintptr_t off = (uintptr_t)below(1 << 16);
    off = below(6) ? off & ~(align - 1) : off | 1;          // mostly aligned
    return reinterpret_cast<void*>(base + off);
}

struct Tally {
    const char* name;
    long seen[8];
    long launched;
};

constexpr int kCalls = 15;
Tally g_tally[kCalls] = {{"nm_spmv", {}, 0},          {"nm_gemv_dense", {}, 0},     {"nm_spmv_multi", {}, 0},
                         {"nm_gemv_dense_multi", {}, 0}, {"nm_spmv_swiglu", {}, 0}, {"nm_gemv_dense_swiglu", {}, 0},
                         {"nm_pack", {}, 0},          {"nm_hybrid_row_loss", {}, 0}, {"nm_hybrid_select_rows", {}, 0},
                         {"nm_hybrid_pack", {}, 0},   {"nm_spmv_hybrid", {}, 0},   {"nm_calib_accumulate", {}, 0},
                         {"nm_calib_keep_mask", {}, 0}, {"nm_spmv_multi_ws", {}, 0}, {"nm_gemv_dense_multi_ws", {}, 0}};

// A workspace pointer and size: usually the right size (256-aligned, in the crowded window or far), sometimes
// too small, misaligned, absent, or an absurd size.
void pick_ws(void** ws, int64_t* bytes)
{
    const int64_t need = nm_workspace_bytes();
    *ws = below(8) ? pick_ptr(256) : nullptr;
    if (*ws && below(4) == 0)
        *ws = reinterpret_cast<void*>(reinterpret_cast<uintptr_t>(*ws) | 16);
    static const int64_t odd[] = {0, 1, -1, INT64_MAX, INT64_MIN};
    const uint64_t r = below(10);
    *bytes = r < 6 ? need : r < 8 ? need - 1 - (int64_t)below(1000) : odd[below(5)];
}

void record(int which, int st, long before)
{
    if (st < 0 || st > 6) {
        std::fprintf(stderr, "%s returned %d, not a status code\n", g_tally[which].name, st);
        std::exit(1);
    }
    ++g_tally[which].seen[st];
    g_tally[which].launched += nmtest_launches() - before;
}

void one_call(int which)
{
    const long before = nmtest_launches();
    const int64_t R = pick_rows(), K = pick_k();
    const int M = pick_m(), N = pick_n(M), B = pick_b(), dt = pick_dtype();
    int st = 0;
    switch (which) {
    case 0:
        st = nm_spmv(pick_ptr(16), (const uint8_t*)pick_ptr(16), R, K, N, M, dt, pick_ptr(16), B, pick_ptr(2), nullptr);
        break;
    case 1: st = nm_gemv_dense(pick_ptr(16), R, K, dt, pick_ptr(16), B, pick_ptr(2), nullptr); break;
    case 2:
    case 3:
    case 13:
    case 14: {
        const int count = below(8) ? 1 + (int)below(4) : (int)below(7) - 1;
        const void* v[6];
        const uint8_t* m[6];
        int64_t Rs[6];
        void* y[6];
        for (int i = 0; i < 6; ++i) {
            v[i] = pick_ptr(16);
            m[i] = (const uint8_t*)pick_ptr(16);
            Rs[i] = below(4) ? (int64_t)below(20) : pick_rows();
            y[i] = pick_ptr(2);
        }
        void* ws = nullptr;
        int64_t wsb = 0;
        pick_ws(&ws, &wsb);
        if (which == 2)
            st = nm_spmv_multi(count, below(20) ? v : nullptr, below(20) ? m : nullptr, below(20) ? Rs : nullptr, K, N,
                               M, dt, pick_ptr(16), B, below(20) ? y : nullptr, nullptr);
        else if (which == 3)
            st = nm_gemv_dense_multi(count, below(20) ? v : nullptr, below(20) ? Rs : nullptr, K, dt, pick_ptr(16), B,
                                     below(20) ? y : nullptr, nullptr);
        else if (which == 13)
            st = nm_spmv_multi_ws(count, below(20) ? v : nullptr, below(20) ? m : nullptr, below(20) ? Rs : nullptr, K,
                                  N, M, dt, pick_ptr(16), B, below(20) ? y : nullptr, ws, wsb, nullptr);
        else
            st = nm_gemv_dense_multi_ws(count, below(20) ? v : nullptr, below(20) ? Rs : nullptr, K, dt, pick_ptr(16),
                                        B, below(20) ? y : nullptr, ws, wsb, nullptr);
        break;
    }
    case 4:
        st = nm_spmv_swiglu(pick_ptr(16), (const uint8_t*)pick_ptr(16), pick_ptr(16), (const uint8_t*)pick_ptr(16), R,
                            K, N, M, dt, pick_ptr(16), B, pick_ptr(2), nullptr);
        break;
    case 5: st = nm_gemv_dense_swiglu(pick_ptr(16), pick_ptr(16), R, K, dt, pick_ptr(16), B, pick_ptr(2), nullptr); break;
    case 6:
        st = nm_pack(pick_ptr(16), below(2) ? (const uint8_t*)pick_ptr(1) : nullptr, R, K, N, M, dt, pick_ptr(16),
                     (uint8_t*)pick_ptr(16), nullptr);
        break;
    case 7: {
        const int64_t hs = below(5) ? 1 + (int64_t)below(50) : (int64_t)below(3) - 1;
        st = nm_hybrid_row_loss(pick_ptr(2), below(2) ? (const uint8_t*)pick_ptr(1) : nullptr,
                                below(2) ? (const float*)pick_ptr(4) : nullptr, hs, R, K, N, M, dt,
                                (double*)pick_ptr(8), nullptr);
        break;
    }
    case 8: {
        const int64_t nd = below(5) ? (R > 0 ? (int64_t)below((uint64_t)(R % 64) + 1) : 0) : pick_rows();
        st = nm_hybrid_select_rows((const double*)pick_ptr(8), R, nd, (uint8_t*)pick_ptr(1), nullptr);
        break;
    }
    case 9:
    case 10: {
        const int64_t nd = below(5) ? (R > 0 ? (int64_t)below((uint64_t)(R % 64) + 1) : 0) : pick_rows();
        if (which == 9)
            st = nm_hybrid_pack(pick_ptr(16), below(2) ? (const uint8_t*)pick_ptr(1) : nullptr,
                                (const uint8_t*)pick_ptr(1), nd, R, K, N, M, dt, pick_ptr(16), (uint8_t*)pick_ptr(16),
                                pick_ptr(16), (int32_t*)pick_ptr(4), (int32_t*)pick_ptr(4), nullptr);
        else
            st = nm_spmv_hybrid(pick_ptr(16), (const uint8_t*)pick_ptr(16), (const int32_t*)pick_ptr(4), pick_ptr(16),
                                (const int32_t*)pick_ptr(4), nd, R, K, N, M, dt, pick_ptr(16), B, pick_ptr(2), nullptr);
        break;
    }
    case 11:
        st = nm_calib_accumulate(pick_ptr(16), below(2) ? (const uint8_t*)pick_ptr(1) : nullptr, R, K, dt,
                                 (float*)pick_ptr(4), nullptr);
        break;
    case 12: {
        const int64_t hs = below(5) ? 1 + (int64_t)below(50) : (int64_t)below(3) - 1;
        st = nm_calib_keep_mask(pick_ptr(16), (const float*)pick_ptr(4), hs, R, K, N, M, dt, (uint8_t*)pick_ptr(8),
                                nullptr);
        break;
    }
    }
    record(which, st, before);
}

}  // namespace

int main(int argc, char** argv)
{
    const long calls = argc > 1 ? std::atol(argv[1]) : 200000;
    for (long i = 0; i < calls; ++i)
        one_call((int)(i % kCalls));
    int bad = 0;
    for (int w = 0; w < kCalls; ++w) {
        const Tally& t = g_tally[w];
        std::printf("%-22s ok %6ld  invalid_arg %6ld  bad_shape %6ld  unsupported %6ld  launched %6ld\n", t.name,
                    t.seen[NM_OK], t.seen[NM_ERR_INVALID_ARG], t.seen[NM_ERR_BAD_SHAPE], t.seen[NM_ERR_UNSUPPORTED],
                    t.launched);
        if (!t.launched || !t.seen[NM_ERR_INVALID_ARG] || !t.seen[NM_ERR_BAD_SHAPE] ||
            !t.seen[NM_ERR_UNSUPPORTED] == (w != 8)) {
            std::fprintf(stderr, "%s: a class of outcome was never reached\n", t.name);
            bad = 1;
        }
    }
    return bad;
}
