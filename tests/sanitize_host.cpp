// sanitize_host.cpp -- host-side checks of libmsscan's C ABI and of the C
// oracle, built with AddressSanitizer and UndefinedBehaviorSanitizer (see
// test_sanitize_host.py).  No GPU is needed: every ABI call here either fails
// validation before anything is launched, or is a pure size query; the oracle
// runs on small host arrays.  Exit status 0 means every check held.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "../include/msscan.h"

extern "C" {
int oracle_scan(const double* u, const double* delta_raw, const double* A, const double* B,
                const double* C, const double* D, const double* z, const double* delta_bias,
                const double* h0, int softplus, int disc, int64_t batch, int64_t L, int64_t Dn,
                int64_t N, double* y, double* h_last, int nthreads);
int oracle_step(double* h, const double* x, const double* delta_raw, const double* A,
                const double* B, const double* C, const double* D, const double* z,
                const double* delta_bias, int softplus, int disc, int64_t batch, int64_t Dn,
                int64_t N, double* y);
int oracle_scan_bwd(const double* u, const double* delta_raw, const double* A, const double* B,
                    const double* C, const double* D, const double* z, const double* delta_bias,
                    const double* h0, int softplus, int disc, int64_t batch, int64_t L,
                    int64_t Dn, int64_t N, const double* dy, const double* dh_last, double* du,
                    double* ddelta, double* dA, double* dB, double* dC, double* dD, double* dz,
                    double* dbias, double* dh0, int nthreads);
int oracle_conv1d(const double* x, const double* w, const double* bias, const double* x_prev,
                  int64_t width, int silu, int64_t batch, int64_t L, int64_t Dn, double* u,
                  int nthreads);
}

static int g_fail = 0;
#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            ++g_fail;                                                      \
        }                                                                  \
    } while (0)

// A fake, 16-byte aligned device address: never dereferenced on these paths.
static void* fake(uintptr_t k) { return reinterpret_cast<void*>(0x100000 + 16 * k); }

static void check_validation() {
    const ms_dims good{2, 100, 64, 16, MS_BF16};
    auto scan = [&](const ms_dims* d, uint32_t flags, const void* u, const void* y,
                    const void* h_last = nullptr) {
        return ms_scan_fwd(u, fake(1), (const float*)fake(2), fake(3), fake(4), nullptr, nullptr,
                           nullptr, flags, const_cast<void*>(y), nullptr, (float*)h_last, d,
                           nullptr, 0, nullptr);
    };
    CHECK(scan(nullptr, 1, fake(0), fake(5)) == MS_ERR_NULL);
    CHECK(scan(&good, 1, nullptr, fake(5)) == MS_ERR_NULL);
    CHECK(std::strlen(ms_last_error()) > 0);
    CHECK(scan(&good, 1, fake(0), nullptr) == MS_ERR_NULL);
    const ms_dims bad_dims[] = {{0, 100, 64, 16, 1},  {1, 0, 64, 16, 1},   {1, 10, 0, 16, 1},
                                {1, 10, 64, 0, 1},    {1, 10, 64, 129, 1}, {-5, 10, 64, 16, 1},
                                {1, -1, 64, 16, 1},   {1, (int64_t)1 << 40, 64, 16, 1}};
    for (const ms_dims& d : bad_dims) CHECK(scan(&d, 1, fake(0), fake(5)) == MS_ERR_SHAPE);
    const ms_dims bad_io{1, 10, 64, 16, 7};
    CHECK(scan(&bad_io, 1, fake(0), fake(5)) == MS_ERR_DTYPE);
    CHECK(scan(&good, 8, fake(0), fake(5)) == MS_ERR_FLAGS);
    CHECK(scan(&good, MS_ZOH | MS_BILINEAR, fake(0), fake(5)) == MS_ERR_FLAGS);
    CHECK(scan(&good, 1, reinterpret_cast<void*>(0x100008), fake(5)) == MS_ERR_ALIGN);
    CHECK(scan(&good, 1, fake(0), fake(5), reinterpret_cast<void*>(0x100004)) == MS_ERR_ALIGN);
    const ms_dims segmented{2, 4096, 64, 16, MS_BF16};  // needs a workspace
    CHECK(ms_scan_workspace_bytes(&segmented, 1) > 0);
    CHECK(scan(&segmented, 1, fake(0), fake(5)) == MS_ERR_WORKSPACE);
    // decode step
    CHECK(ms_state_update((float*)fake(0), fake(1), fake(2), (const float*)fake(3), fake(4),
                          fake(5), nullptr, nullptr, nullptr, 1, fake(6), 0, 64, 16, 1,
                          nullptr) == MS_ERR_SHAPE);
    CHECK(ms_state_update(nullptr, fake(1), fake(2), (const float*)fake(3), fake(4), fake(5),
                          nullptr, nullptr, nullptr, 1, fake(6), 1, 64, 16, 1,
                          nullptr) == MS_ERR_NULL);
    CHECK(ms_state_update((float*)fake(0), fake(1), fake(2), (const float*)fake(3), fake(4),
                          fake(5), nullptr, nullptr, nullptr, 6, fake(6), 1, 64, 16, 1,
                          nullptr) == MS_ERR_FLAGS);
    // conv1d
    CHECK(ms_conv1d_silu(fake(0), (const float*)fake(1), nullptr, nullptr, 9, 1, fake(2), 2, 10,
                         8, 1, nullptr) == MS_ERR_SHAPE);
    CHECK(ms_conv1d_silu(nullptr, (const float*)fake(1), nullptr, nullptr, 4, 1, fake(2), 2, 10,
                         8, 1, nullptr) == MS_ERR_NULL);
    // backward
    const ms_dims n32{1, 64, 64, 200, MS_F32};
    CHECK(ms_scan_bwd(fake(0), fake(1), (const float*)fake(2), fake(3), fake(4), nullptr, nullptr,
                      nullptr, 1, nullptr, fake(5), nullptr, fake(6), fake(7), (float*)fake(8),
                      (float*)fake(9), (float*)fake(10), nullptr, nullptr, nullptr, nullptr,
                      &n32, fake(11), 1 << 20, nullptr) == MS_ERR_SHAPE);
    CHECK(ms_scan_bwd(fake(0), fake(1), (const float*)fake(2), fake(3), fake(4), nullptr,
                      fake(12), nullptr, 1, nullptr, fake(5), nullptr, fake(6), fake(7),
                      (float*)fake(8), (float*)fake(9), (float*)fake(10), nullptr, nullptr,
                      nullptr, nullptr, &good, fake(11), 1 << 20, nullptr) == MS_ERR_NULL);
    // fused step projection
    CHECK(ms_scan_fwd_dtproj(fake(0), fake(1), fake(2), 0, (const float*)fake(3), fake(4),
                             fake(5), nullptr, nullptr, nullptr, 1, fake(6), nullptr, nullptr,
                             &good, nullptr, 0, nullptr) == MS_ERR_SHAPE);
    // checkpointed pair: required checkpoint, a shape it does not serve
    CHECK(ms_scan_fwd_checkpoint(fake(0), fake(1), (const float*)fake(2), fake(3), fake(4),
                                 nullptr, nullptr, nullptr, 1, fake(5), nullptr, nullptr, nullptr,
                                 &good, nullptr) == MS_ERR_NULL);
    CHECK(ms_scan_fwd_checkpoint(fake(0), fake(1), (const float*)fake(2), fake(3), fake(4),
                                 nullptr, nullptr, nullptr, 1, fake(5), nullptr, nullptr,
                                 (float*)fake(6), &good, nullptr) == MS_ERR_UNSUPPORTED);
    CHECK(ms_scan_bwd_checkpoint(fake(0), fake(1), (const float*)fake(2), fake(3), fake(4),
                                 nullptr, nullptr, nullptr, 1, (const float*)fake(5), fake(6),
                                 nullptr, fake(7), fake(8), (float*)fake(9), (float*)fake(10),
                                 (float*)fake(11), nullptr, nullptr, nullptr, nullptr, &good,
                                 fake(12), 1 << 20, nullptr) == MS_ERR_UNSUPPORTED);
    // conv workgroup count beyond the grid
    CHECK(ms_conv1d_silu(fake(0), (const float*)fake(1), nullptr, nullptr, 4, 1, fake(2), 65535,
                         0x7fffffff, 4, 1, nullptr) == MS_ERR_UNSUPPORTED);
    // sizes whose product leaves size_t's comfortable range
    const ms_dims huge{65535, 0x7fffffff, 1 << 20, 128, MS_BF16};
    CHECK(scan(&huge, 1, fake(0), fake(5)) == MS_ERR_SHAPE);
    CHECK(ms_scan_workspace_bytes(&huge, 1) == (size_t)-1);
    // status strings
    for (int s = 0; s <= 9; ++s) CHECK(ms_status_string((ms_status)s) != nullptr);
    CHECK(ms_abi_version() == MS_ABI_VERSION);
    // profile: closed; bad counts
    CHECK(ms_profile_end(nullptr) == MS_ERR_UNSUPPORTED);
    CHECK(ms_profile_begin(0) == MS_ERR_SHAPE);
    CHECK(ms_profile_begin(5000) == MS_ERR_SHAPE);
}

// The planners' size arithmetic over a grid of shapes, flags and io types:
// sizes are multiples of 256 (or 0, or the invalid marker) and grow with L.
static void check_workspace_sizes() {
    const int32_t batches[] = {1, 2, 7, 64, 65535};
    const int64_t lens[] = {1, 15, 16, 17, 255, 4096, 1 << 20, 0x7fffffff};
    const int32_t dins[] = {1, 8, 63, 64, 65, 1536, 5120, 262144};
    const int32_t states[] = {1, 4, 8, 9, 15, 16, 17, 31, 32, 33, 48, 64, 65, 100, 128};
    for (int32_t b : batches)
        for (int64_t L : lens)
            for (int32_t D : dins)
                for (int32_t N : states)
                    for (uint32_t f : {0u, 1u, 2u, 3u, 4u, 5u})
                        for (int32_t io : {0, 1}) {
                            const ms_dims d{b, L, D, N, io};
                            const size_t ws = ms_scan_workspace_bytes(&d, f);
                            CHECK(ws == (size_t)-1 || ws % 256 == 0);
                            const size_t wd = ms_scan_dtproj_workspace_bytes(&d, f);
                            CHECK(wd == (size_t)-1 || wd % 256 == 0);
                            const size_t wb = ms_scan_bwd_workspace_bytes(&d, f);
                            CHECK(wb == (size_t)-1 || wb % 4 == 0);
                            const size_t ck = ms_scan_checkpoint_bytes(&d, f);
                            CHECK(ck == (size_t)-1 || ck % 256 == 0);
                            const size_t wc = ms_scan_bwd_checkpoint_workspace_bytes(&d, f);
                            CHECK((ck == 0 || ck == (size_t)-1) ? wc == (size_t)-1
                                                                : wc == wb - ck);
                        }
    const ms_dims a{1, 65536, 256, 16, 1}, c{1, 2 * 65536, 256, 16, 1};
    CHECK(ms_scan_workspace_bytes(&c, 1) >= ms_scan_workspace_bytes(&a, 1));
}

// The oracle on small random inputs, every discretisation and option.
static void check_oracle() {
    std::mt19937 rng(7);
    std::normal_distribution<double> nd(0.0, 1.0);
    const int64_t Bt = 2, L = 37, Dn = 5, N = 6, W = 4;
    auto vec = [&](size_t n, double s = 1.0) {
        std::vector<double> v(n);
        for (double& x : v) x = s * nd(rng);
        return v;
    };
    std::vector<double> u = vec(Bt * L * Dn), dl = vec(Bt * L * Dn, 0.5), z = vec(Bt * L * Dn);
    std::vector<double> Bm = vec(Bt * L * N), Cm = vec(Bt * L * N), D = vec(Dn), bias = vec(Dn, 0.3);
    std::vector<double> A(Dn * N), h0 = vec(Bt * Dn * N), dy = vec(Bt * L * Dn);
    for (int64_t i = 0; i < Dn * N; ++i) A[i] = -std::exp(0.2 * (double)(i % N));
    A[3] = 0.0;  // the ZOH limit branch
    for (int disc = 0; disc < 3; ++disc)
        for (int sp = 0; sp < 2; ++sp) {
            std::vector<double> y(Bt * L * Dn), hl(Bt * Dn * N);
            CHECK(oracle_scan(u.data(), dl.data(), A.data(), Bm.data(), Cm.data(), D.data(),
                              z.data(), bias.data(), h0.data(), sp, disc, Bt, L, Dn, N, y.data(),
                              hl.data(), 2) == 0);
            for (double v : y) CHECK(std::isfinite(v));
            std::vector<double> h(h0), ys(Bt * Dn);
            std::vector<double> xt(Bt * Dn), dt(Bt * Dn), zt(Bt * Dn), bt(Bt * N), ct(Bt * N);
            for (int64_t b = 0; b < Bt; ++b) {
                for (int64_t d = 0; d < Dn; ++d) {
                    xt[b * Dn + d] = u[b * L * Dn + d];
                    dt[b * Dn + d] = dl[b * L * Dn + d];
                    zt[b * Dn + d] = z[b * L * Dn + d];
                }
                for (int64_t n = 0; n < N; ++n) {
                    bt[b * N + n] = Bm[b * L * N + n];
                    ct[b * N + n] = Cm[b * L * N + n];
                }
            }
            CHECK(oracle_step(h.data(), xt.data(), dt.data(), A.data(), bt.data(), ct.data(),
                              D.data(), zt.data(), bias.data(), sp, disc, Bt, Dn, N,
                              ys.data()) == 0);
            for (int64_t b = 0; b < Bt; ++b)  // one step equals the scan's first step
                for (int64_t d = 0; d < Dn; ++d)
                    CHECK(std::fabs(ys[b * Dn + d] - y[b * L * Dn + d]) <= 1e-12 * (1 + std::fabs(ys[b * Dn + d])));
            std::vector<double> du(u.size()), ddl(u.size()), dz(u.size()), dA(A.size()),
                dB(Bm.size()), dC(Cm.size()), dD(Dn), db(Dn), dh0(h0.size());
            CHECK(oracle_scan_bwd(u.data(), dl.data(), A.data(), Bm.data(), Cm.data(), D.data(),
                                  z.data(), bias.data(), h0.data(), sp, disc, Bt, L, Dn, N,
                                  dy.data(), h0.data(), du.data(), ddl.data(), dA.data(),
                                  dB.data(), dC.data(), dD.data(), dz.data(), db.data(),
                                  dh0.data(), 2) == 0);
            for (double v : dA) CHECK(std::isfinite(v));
        }
    std::vector<double> w = vec(Dn * W, 0.5), cb = vec(Dn, 0.1), xp = vec(Bt * (W - 1) * Dn), uo(u.size());
    CHECK(oracle_conv1d(u.data(), w.data(), cb.data(), xp.data(), W, 1, Bt, L, Dn, uo.data(), 2) == 0);
    for (double v : uo) CHECK(std::isfinite(v));
    CHECK(oracle_scan(nullptr, dl.data(), A.data(), Bm.data(), Cm.data(), nullptr, nullptr,
                      nullptr, nullptr, 1, 0, Bt, L, Dn, N, u.data(), nullptr, 1) != 0);
}

int main() {
    check_validation();
    check_workspace_sizes();
    check_oracle();
    if (g_fail) {
        std::fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    std::printf("sanitized host checks passed\n");
    return 0;
}
