// launch_stub.cpp -- a CPU stand-in for libnmspmv's kernel side (nm_launch.h),
// linked with the real entry points (nmapi.cpp) so that their checks build
// and run without HIP, under sanitizers.  Each call first checks what
// nm_launch.h promises the kernels -- shapes in range, pointers present and
// aligned, every output disjoint from every input and from the other outputs
// -- written out here from the header's rules, not with nm_rules.h; a broken
// promise prints the call and aborts.  Then it counts itself and returns
// NM_ERR_HIP: there is no GPU behind it.  nmtest_launches() returns the count.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "nm_launch.h"
#include "nmspmv.h"

namespace {

long g_launches = 0;
const int64_t kRows = (int64_t(1) << 31) - 1024;   // rows (and a gated call's 2 R) stay below this

void promise(bool ok, const char* call, const char* what)
{
    if (!ok) {
        std::fprintf(stderr, "kernel precondition broken: %s: %s\n", call, what);
        std::abort();
    }
}

bool al(const void* p, uintptr_t a) { return p != nullptr && reinterpret_cast<uintptr_t>(p) % a == 0; }

struct Buf {
    const void* p;
    uint64_t n;
};

// [p, p + n) and [q, q + m) share no byte (empty buffers share none).
bool apart(Buf a, Buf b)
{
    if (a.n == 0 || b.n == 0 || !a.p || !b.p)
        return true;
    const unsigned __int128 a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 + a.n <= b0 || b0 + b.n <= a0;
}

void outputs_apart(const char* call, const std::vector<Buf>& outs, const std::vector<Buf>& ins)
{
    for (size_t i = 0; i < outs.size(); ++i) {
        for (const Buf& in : ins)
            promise(apart(outs[i], in), call, "an output overlaps an input");
        for (size_t j = i + 1; j < outs.size(); ++j)
            promise(apart(outs[i], outs[j]), call, "two outputs overlap");
    }
}

void shape(const char* call, int64_t R, int64_t K, bool kpos, int dtype)
{
    promise(R > 0 && R < kRows, call, "R out of range");
    promise(K >= 0 && K <= INT32_MAX && K % 8 == 0 && (!kpos || K > 0), call, "K out of range");
    promise(dtype == NM_FP16 || dtype == NM_BF16, call, "dtype");
}

void nm(const char* call, int64_t K, int N, int M)
{
    promise((M == 4 || M == 8) && N >= 1 && N < M && K % M == 0, call, "N:M");
}

void batch(const char* call, int B) { promise(B >= 1 && B <= 32, call, "B out of range"); }

int launched()
{
    ++g_launches;
    return NM_ERR_HIP;
}

}  // namespace

extern "C" long nmtest_launches(void) { return g_launches; }

// The library's allocation-free workspace: here a fixed, 256-byte aligned stand-in address (never dereferenced).
int nmk::static_workspace(void** out, void*)
{
    *out = reinterpret_cast<void*>(uintptr_t(0x7f0000000000));
    return NM_OK;
}

int nmk::zero(void* y, int64_t n, void*)
{
    promise(n > 0 && al(y, 2), "zero", "y");
    return launched();
}

// A workspace, when given, is ws_bytes (the library's constant) long, 256-byte aligned and apart from every
// input and output.
void workspace(const char* c, const void* ws, const std::vector<Buf>& ins, const std::vector<Buf>& outs)
{
    if (!ws)
        return;
    promise(reinterpret_cast<uintptr_t>(ws) % 256 == 0, c, "workspace alignment");
    const Buf w{ws, (uint64_t)nm_workspace_bytes()};
    for (const Buf& b : ins)
        promise(apart(w, b), c, "workspace overlaps an input");
    for (const Buf& b : outs)
        promise(apart(w, b), c, "workspace overlaps an output");
}

int nmk::spmv_multi(int count, const void* const* values, const uint8_t* const* masks, const int64_t* R, int64_t total,
                    int64_t K, int N, int M, int dtype, const void* x, int B, void* const* y, void* ws, void*)
{
    const char* c = "spmv_multi";
    promise(count >= 1 && count <= 4 && values && masks && R && y, c, "part arrays");
    int64_t sum = 0;
    for (int i = 0; i < count; ++i) {
        promise(R[i] >= 0 && R[i] < kRows, c, "R[i]");
        sum += R[i];
    }
    promise(sum == total, c, "total");
    shape(c, total, K, true, dtype);
    nm(c, K, N, M);
    batch(c, B);
    promise(al(x, 16), c, "x");
    std::vector<Buf> ins{{x, (uint64_t)B * K * 2}}, outs;
    for (int i = 0; i < count; ++i) {
        if (R[i] == 0)
            continue;
        promise(al(values[i], 16) && al(masks[i], 16) && al(y[i], 2), c, "part pointers");
        ins.push_back({values[i], (uint64_t)R[i] * (K / M * N) * 2});
        ins.push_back({masks[i], (uint64_t)R[i] * (K / 8)});
        outs.push_back({y[i], (uint64_t)B * R[i] * 2});
    }
    outputs_apart(c, outs, ins);
    workspace(c, ws, ins, outs);
    return launched();
}

int nmk::gemv_dense_multi(int count, const void* const* W, const int64_t* R, int64_t total, int64_t K, int dtype,
                          const void* x, int B, void* const* y, void* ws, void*)
{
    const char* c = "gemv_dense_multi";
    promise(count >= 1 && count <= 4 && W && R && y, c, "part arrays");
    int64_t sum = 0;
    for (int i = 0; i < count; ++i) {
        promise(R[i] >= 0 && R[i] < kRows, c, "R[i]");
        sum += R[i];
    }
    promise(sum == total, c, "total");
    shape(c, total, K, true, dtype);
    batch(c, B);
    promise(al(x, 16), c, "x");
    std::vector<Buf> ins{{x, (uint64_t)B * K * 2}}, outs;
    for (int i = 0; i < count; ++i) {
        if (R[i] == 0)
            continue;
        promise(al(W[i], 16) && al(y[i], 2), c, "part pointers");
        ins.push_back({W[i], (uint64_t)R[i] * K * 2});
        outs.push_back({y[i], (uint64_t)B * R[i] * 2});
    }
    outputs_apart(c, outs, ins);
    workspace(c, ws, ins, outs);
    return launched();
}

int nmk::spmv_swiglu(const void* vg, const uint8_t* mg, const void* vu, const uint8_t* mu, int64_t R, int64_t K, int N,
                     int M, int dtype, const void* x, int B, void* h, void*)
{
    const char* c = "spmv_swiglu";
    shape(c, R, K, true, dtype);
    promise(2 * R < kRows, c, "2 R");
    nm(c, K, N, M);
    batch(c, B);
    promise(al(vg, 16) && al(mg, 16) && al(vu, 16) && al(mu, 16) && al(x, 16) && al(h, 2), c, "pointers");
    const uint64_t vb = (uint64_t)R * (K / M * N) * 2, mb = (uint64_t)R * (K / 8);
    outputs_apart(c, {{h, (uint64_t)B * R * 2}}, {{vg, vb}, {mg, mb}, {vu, vb}, {mu, mb}, {x, (uint64_t)B * K * 2}});
    return launched();
}

int nmk::gemv_dense_swiglu(const void* Wg, const void* Wu, int64_t R, int64_t K, int dtype, const void* x, int B,
                           void* h, void*)
{
    const char* c = "gemv_dense_swiglu";
    shape(c, R, K, true, dtype);
    promise(2 * R < kRows, c, "2 R");
    batch(c, B);
    promise(al(Wg, 16) && al(Wu, 16) && al(x, 16) && al(h, 2), c, "pointers");
    const uint64_t wb = (uint64_t)R * K * 2;
    outputs_apart(c, {{h, (uint64_t)B * R * 2}}, {{Wg, wb}, {Wu, wb}, {x, (uint64_t)B * K * 2}});
    return launched();
}

int nmk::pack(const void* W, const uint8_t* keep, int64_t R, int64_t K, int N, int M, int dtype, void* values,
              uint8_t* masks, void*)
{
    const char* c = "pack";
    shape(c, R, K, true, dtype);
    nm(c, K, N, M);
    promise(al(W, 16) && al(values, 16) && al(masks, 16), c, "pointers");
    outputs_apart(c, {{values, (uint64_t)R * (K / M * N) * 2}, {masks, (uint64_t)R * (K / 8)}},
                  {{W, (uint64_t)R * K * 2}, {keep, keep ? (uint64_t)R * K : 0}});
    return launched();
}

int nmk::hybrid_row_loss(const void* W, const uint8_t* keep, const float* h, int64_t h_stride, int64_t R, int64_t K,
                         int N, int M, int dtype, double* loss, void*)
{
    const char* c = "hybrid_row_loss";
    shape(c, R, K, false, dtype);
    nm(c, K, N, M);
    promise((K == 0 || al(W, 2)) && al(loss, 8) && (!h || h_stride >= 1) && (!h || K == 0 || al(h, 4)), c, "pointers");
    const uint64_t hb = h && K > 0 ? ((uint64_t)(K - 1) * h_stride + 1) * 4 : 0;
    outputs_apart(c, {{loss, (uint64_t)R * 8}}, {{W, (uint64_t)R * K * 2}, {keep, keep ? (uint64_t)R * K : 0}, {h, hb}});
    return launched();
}

int nmk::hybrid_select_rows(const double* loss, int64_t R, int64_t n_dense, uint8_t* flags, void*)
{
    const char* c = "hybrid_select_rows";
    promise(R > 0 && R < kRows && n_dense >= 0 && n_dense <= R, c, "shape");
    promise(al(loss, 8) && flags, c, "pointers");
    outputs_apart(c, {{flags, (uint64_t)R}}, {{loss, (uint64_t)R * 8}});
    return launched();
}

int nmk::hybrid_pack(const void* W, const uint8_t* keep, const uint8_t* flags, int64_t n_dense, int64_t R, int64_t K,
                     int N, int M, int dtype, void* values, uint8_t* masks, void* W_dense, int32_t* rows_sparse,
                     int32_t* rows_dense, void*)
{
    const char* c = "hybrid_pack";
    shape(c, R, K, false, dtype);
    nm(c, K, N, M);
    promise(n_dense >= 0 && n_dense <= R, c, "n_dense");
    const int64_t Rs = R - n_dense;
    const uint64_t vb = (uint64_t)Rs * (K / M * N) * 2, mb = (uint64_t)Rs * (K / 8), db = (uint64_t)n_dense * K * 2;
    promise((K == 0 || al(W, 16)) && flags, c, "inputs");      // K = 0: W holds no bytes and may be NULL
    promise((vb == 0 || al(values, 16)) && (mb == 0 || al(masks, 16)) && (db == 0 || al(W_dense, 16)) &&
                (Rs == 0 || al(rows_sparse, 4)) && (n_dense == 0 || al(rows_dense, 4)),
            c, "outputs");
    outputs_apart(c, {{values, vb}, {masks, mb}, {W_dense, db}, {rows_sparse, (uint64_t)Rs * 4},
                      {rows_dense, (uint64_t)n_dense * 4}},
                  {{W, (uint64_t)R * K * 2}, {keep, keep ? (uint64_t)R * K : 0}, {flags, (uint64_t)R}});
    return launched();
}

int nmk::spmv_hybrid(const void* values, const uint8_t* masks, const int32_t* rows_sparse, const void* W_dense,
                     const int32_t* rows_dense, int64_t n_dense, int64_t R, int64_t K, int N, int M, int dtype,
                     const void* x, int B, void* y, void*)
{
    const char* c = "spmv_hybrid";
    shape(c, R, K, true, dtype);
    nm(c, K, N, M);
    batch(c, B);
    promise(n_dense >= 0 && n_dense <= R, c, "n_dense");
    const int64_t Rs = R - n_dense;
    const uint64_t vb = (uint64_t)Rs * (K / M * N) * 2, mb = (uint64_t)Rs * (K / 8), db = (uint64_t)n_dense * K * 2;
    promise((vb == 0 || al(values, 16)) && (mb == 0 || al(masks, 16)) && (db == 0 || al(W_dense, 16)) &&
                (Rs == 0 || al(rows_sparse, 4)) && (n_dense == 0 || al(rows_dense, 4)) && al(x, 16) && al(y, 2),
            c, "pointers");
    outputs_apart(c, {{y, (uint64_t)B * R * 2}},
                  {{values, vb}, {masks, mb}, {W_dense, db}, {rows_sparse, (uint64_t)Rs * 4},
                   {rows_dense, (uint64_t)n_dense * 4}, {x, (uint64_t)B * K * 2}});
    return launched();
}

int nmk::calib_accumulate(const void* X, const uint8_t* decode, int64_t T, int64_t K, int dtype, float* H, void*)
{
    const char* c = "calib_accumulate";
    promise(T > 0 && T <= INT32_MAX && K > 0 && K <= 65536 && K % 8 == 0, c, "shape");
    promise(dtype == NM_FP16 || dtype == NM_BF16, c, "dtype");
    promise(al(X, 16) && al(H, 4), c, "pointers");
    outputs_apart(c, {{H, (uint64_t)K * K * 4}}, {{X, (uint64_t)T * K * 2}, {decode, decode ? (uint64_t)T : 0}});
    return launched();
}

int nmk::calib_keep_mask(const void* W, const float* h, int64_t h_stride, int64_t R, int64_t K, int N, int M, int dtype,
                         uint8_t* keep, void*)
{
    const char* c = "calib_keep_mask";
    shape(c, R, K, true, dtype);
    nm(c, K, N, M);
    promise(h_stride >= 1 && al(W, 16) && al(keep, 8) && al(h, 4), c, "pointers");
    outputs_apart(c, {{keep, (uint64_t)R * K}}, {{W, (uint64_t)R * K * 2}, {h, ((uint64_t)(K - 1) * h_stride + 1) * 4}});
    return launched();
}
