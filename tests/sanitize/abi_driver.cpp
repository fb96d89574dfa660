// Host-side check of the C ABI's argument validation under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py, no GPU needed).
//
// csrc/kda_abi.cpp is compiled for the host only and linked against the stand-ins below: every
// kernel launcher records its arguments and returns hipSuccess, and the two HIP runtime calls the
// validation mode makes (hipMemcpyAsync, hipStreamSynchronize) copy host memory.  Every buffer
// the driver passes is host memory of exactly the size the call may touch, so that a read past
// the end in the validation code is reported by the sanitizer.  Exit status 0 when every
// expectation holds; the first failed one is printed.
#include "kda.h"
#include "kda_internal.h"

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace {
int g_launches = 0;               // launcher calls since the last reset
const char* g_last = "";          // name of the last launcher called
kda::PrefillArgs g_prefill;       // arguments of the last prefill launch
kda::DecodeArgs g_decode;         // arguments of the last decode launch
int64_t g_c64_chunks = -1;

void reset() {
    g_launches = 0;
    g_last = "";
    g_c64_chunks = -1;
}
}  // namespace

namespace kda {
hipError_t launch_prefill_general(const PrefillArgs& a, hipStream_t) {
    ++g_launches; g_last = "general"; g_prefill = a; return hipSuccess;
}
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t) {
    ++g_launches; g_last = "mfma"; g_prefill = a; return hipSuccess;
}
hipError_t launch_prefill_c64(const PrefillArgs& a, hipStream_t) {
    ++g_launches; g_last = "c64"; g_prefill = a; return hipSuccess;
}
hipError_t launch_split_finish(const PrefillArgs& a, hipStream_t) {
    ++g_launches; g_last = "split_finish"; g_prefill = a; return hipSuccess;
}
hipError_t launch_decode_d128(const DecodeArgs& a, hipStream_t) {
    ++g_launches; g_last = "decode_d128"; g_decode = a; return hipSuccess;
}
hipError_t launch_output_gate(const GateArgs&, hipStream_t) {
    ++g_launches; g_last = "output_gate"; return hipSuccess;
}
hipError_t launch_frontend(const FrontArgs&, hipStream_t) {
    ++g_launches; g_last = "frontend"; return hipSuccess;
}
size_t c64_mfma_workspace_bytes(int64_t nchunks, int64_t N, int64_t H) {
    return static_cast<size_t>(nchunks) * H * 1024 + static_cast<size_t>(N + 1) * 8;
}
hipError_t launch_prefill_c64_mfma(const PrefillArgs& a, void*, int64_t nchunks, hipStream_t) {
    ++g_launches; g_last = "c64_mfma"; g_prefill = a; g_c64_chunks = nchunks; return hipSuccess;
}
}  // namespace kda

extern "C" hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind,
                                     hipStream_t) {
    std::memcpy(dst, src, bytes);
    return hipSuccess;
}
extern "C" hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

namespace {
int g_failures = 0;

#define EXPECT(cond)                                                                  \
    do {                                                                              \
        if (!(cond)) {                                                                \
            std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, \
                         #cond);                                                      \
            ++g_failures;                                                             \
        }                                                                             \
    } while (0)

// A prefill problem with host buffers of the exact sizes the kernels would touch.
struct Prefill {
    int B, T, H, dk, dv, dtype;
    std::vector<int32_t> cu;           // empty: equal-length batch
    std::vector<unsigned char> q, k, v, g, beta, o;
    std::vector<float> h0, hT;
    Prefill(int B_, int T_, int H_, int dk_, int dv_, int dtype_, std::vector<int32_t> cu_ = {})
        : B(B_), T(T_), H(H_), dk(dk_), dv(dv_), dtype(dtype_), cu(std::move(cu_)) {
        const size_t es = dtype == KDA_BF16 ? 2 : 4;
        const size_t N = cu.empty() ? B : cu.size() - 1;
        const size_t Tt = cu.empty() ? static_cast<size_t>(B) * T : T;
        q.assign(Tt * H * dk * es, 0);
        k.assign(Tt * H * dk * es, 0);
        g.assign(Tt * H * dk * es, 0);
        v.assign(Tt * H * dv * es, 0);
        o.assign(Tt * H * dv * es, 0);
        beta.assign(Tt * H * es, 0);
        h0.assign(N * H * dk * dv, 0.f);
        hT.assign(N * H * dk * dv, 0.f);
    }
    const int32_t* cup() const { return cu.empty() ? nullptr : cu.data(); }
    int nseq() const { return cu.empty() ? 0 : static_cast<int>(cu.size()) - 1; }
    int run() {
        return kda_chunk_fwd(q.data(), k.data(), v.data(), g.data(), beta.data(), h0.data(),
                             cup(), nseq(), o.data(), hT.data(), B, T, H, dk, dv, dtype, nullptr);
    }
};

void set_validate(bool on) {
    if (on) setenv("KDA_VALIDATE", "1", 1);
    else unsetenv("KDA_VALIDATE");
}

// bf16 bit patterns of a few g values
uint16_t bf16_of(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    return static_cast<uint16_t>(u >> 16);
}

void test_status_strings() {
    for (int s = -20; s <= 5; ++s) EXPECT(kda_status_string(s) != nullptr);
    EXPECT(std::strcmp(kda_status_string(KDA_OK), "ok") == 0);
    EXPECT(kda_version() > 0);
}

void test_prefill_dispatch() {
    {
        reset();
        Prefill p(2, 40, 3, 128, 128, KDA_BF16);
        EXPECT(p.run() == KDA_OK);
        EXPECT(g_launches == 1 && std::strcmp(g_last, "mfma") == 0);
        EXPECT(g_prefill.N == 2 && g_prefill.T == 40 && g_prefill.H == 3);
    }
    {
        reset();
        Prefill p(1, 40, 2, 64, 32, KDA_F32);
        EXPECT(p.run() == KDA_OK);
        EXPECT(g_launches == 1 && std::strcmp(g_last, "general") == 0);
    }
    {
        reset();   // varlen: T is the packed total, the kernel gets T = 0 and cu_seqlens
        Prefill p(1, 50, 2, 128, 128, KDA_BF16, {0, 17, 17, 50});
        EXPECT(p.run() == KDA_OK);
        EXPECT(g_launches == 1 && g_prefill.N == 3 && g_prefill.T == 0 && g_prefill.cu);
    }
    {
        reset();   // empty batch: nothing runs
        Prefill p(0, 40, 2, 128, 128, KDA_BF16);
        EXPECT(p.run() == KDA_OK && g_launches == 0);
    }
    {
        reset();   // zero tokens still writes hT (= h0)
        Prefill p(2, 0, 2, 128, 128, KDA_BF16);
        EXPECT(p.run() == KDA_OK && g_launches == 1);
    }
}

void test_prefill_rejects() {
    Prefill p(1, 32, 2, 128, 128, KDA_BF16);
    auto call = [&](const void* q, int B, int T, int H, int dk, int dv, int dtype,
                    const int32_t* cu = nullptr, int ns = 0) {
        reset();
        const int st = kda_chunk_fwd(q, p.k.data(), p.v.data(), p.g.data(), p.beta.data(),
                                     p.h0.data(), cu, ns, p.o.data(), p.hT.data(), B, T, H, dk,
                                     dv, dtype, nullptr);
        EXPECT(g_launches == 0);   // nothing runs on an argument error
        return st;
    };
    EXPECT(call(p.q.data(), 1, 32, 2, 128, 128, 7) == KDA_ERR_DTYPE);
    EXPECT(call(p.q.data(), -1, 32, 2, 128, 128, KDA_BF16) == KDA_ERR_SHAPE);
    EXPECT(call(p.q.data(), 1, -5, 2, 128, 128, KDA_BF16) == KDA_ERR_SHAPE);
    EXPECT(call(p.q.data(), 1, 32, 0, 128, 128, KDA_BF16) == KDA_ERR_SHAPE);
    EXPECT(call(p.q.data(), 1, 32, 2, 120, 128, KDA_BF16) == KDA_ERR_UNSUPPORTED);
    EXPECT(call(p.q.data(), 1, 32, 2, 128, 144, KDA_BF16) == KDA_ERR_UNSUPPORTED);
    EXPECT(call(p.q.data(), 1, 32, 2, 0, 128, KDA_BF16) == KDA_ERR_UNSUPPORTED);
    EXPECT(call(nullptr, 1, 32, 2, 128, 128, KDA_BF16) == KDA_ERR_NULL);
    // a token row of more than 2^20 elements
    EXPECT(call(p.q.data(), 1, 32, 8193, 128, 128, KDA_BF16) == KDA_ERR_SHAPE);
    // cu_seqlens needs B == 1
    const std::vector<int32_t> cu = {0, 32};
    EXPECT(call(p.q.data(), 2, 32, 2, 128, 128, KDA_BF16, cu.data(), 1) == KDA_ERR_SEQLENS);
    // sizes whose products overflow 32 bits are still only compared, never used unchecked
    reset();
    EXPECT(kda_chunk_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                         nullptr, nullptr, 2147483647, 2147483647, 64, 128, 128, KDA_BF16,
                         nullptr) == KDA_ERR_NULL);
    EXPECT(g_launches == 0);
}

void test_validate_mode() {
    set_validate(true);
    {
        reset();   // good contents pass
        Prefill p(1, 40, 2, 128, 128, KDA_BF16, {0, 8, 40});
        const uint16_t m5 = bf16_of(-5.0f), m1 = bf16_of(-1.0f);
        uint16_t* gb = reinterpret_cast<uint16_t*>(p.g.data());
        for (size_t i = 0; i < p.g.size() / 2; ++i) gb[i] = (i % 2) ? m5 : m1;
        EXPECT(p.run() == KDA_OK && g_launches == 1);
        gb[p.g.size() / 2 - 1] = bf16_of(-5.5f);   // the last element, below the floor
        reset();
        EXPECT(p.run() == KDA_ERR_RANGE && g_launches == 0);
        gb[0] = bf16_of(0.25f);
        reset();
        EXPECT(p.run() == KDA_ERR_RANGE && g_launches == 0);
    }
    {
        Prefill p(1, 40, 2, 64, 64, KDA_F32, {0, 30, 20, 40});   // decreasing
        reset();
        EXPECT(p.run() == KDA_ERR_SEQLENS && g_launches == 0);
    }
    {
        Prefill p(1, 40, 2, 64, 64, KDA_F32, {0, 8, 39});   // does not end at T
        reset();
        EXPECT(p.run() == KDA_ERR_SEQLENS && g_launches == 0);
    }
    {
        Prefill p(1, 40, 2, 64, 64, KDA_F32, {1, 8, 40});   // does not start at 0
        reset();
        EXPECT(p.run() == KDA_ERR_SEQLENS && g_launches == 0);
    }
    {
        // snapshot offsets must match the lengths: sequence lengths 32 and 16 at stride 16 give
        // 2 and 1 snapshots
        Prefill p(1, 48, 1, 32, 32, KDA_F32, {0, 32, 48});
        std::vector<float> snaps(3 * 32 * 32);
        std::vector<int32_t> good = {0, 2, 3}, bad = {0, 1, 3};
        reset();
        EXPECT(kda_chunk_fwd_snapshots(p.q.data(), p.k.data(), p.v.data(), p.g.data(),
                                       p.beta.data(), p.h0.data(), p.cup(), 2, p.o.data(),
                                       p.hT.data(), snaps.data(), good.data(), 16, 1, 48, 1, 32,
                                       32, KDA_F32, nullptr) == KDA_OK);
        EXPECT(g_launches == 1 && g_prefill.snaps && g_prefill.snap_tiles == 1);
        reset();
        EXPECT(kda_chunk_fwd_snapshots(p.q.data(), p.k.data(), p.v.data(), p.g.data(),
                                       p.beta.data(), p.h0.data(), p.cup(), 2, p.o.data(),
                                       p.hT.data(), snaps.data(), bad.data(), 16, 1, 48, 1, 32,
                                       32, KDA_F32, nullptr) == KDA_ERR_STRIDE);
        EXPECT(g_launches == 0);
    }
    set_validate(false);
}

void test_snapshots_args() {
    Prefill p(1, 64, 1, 32, 32, KDA_F32);
    std::vector<float> snaps(4 * 32 * 32);
    auto call = [&](int stride, float* s) {
        reset();
        return kda_chunk_fwd_snapshots(p.q.data(), p.k.data(), p.v.data(), p.g.data(),
                                       p.beta.data(), p.h0.data(), nullptr, 0, p.o.data(),
                                       p.hT.data(), s, nullptr, stride, 1, 64, 1, 32, 32, KDA_F32,
                                       nullptr);
    };
    EXPECT(call(0, snaps.data()) == KDA_ERR_STRIDE);
    EXPECT(call(-16, snaps.data()) == KDA_ERR_STRIDE);
    EXPECT(call(24, snaps.data()) == KDA_ERR_STRIDE);
    EXPECT(call(16, nullptr) == KDA_ERR_NULL);
    EXPECT(call(16, snaps.data()) == KDA_OK && g_prefill.snap_per_seq == 4);
    EXPECT(call(128, nullptr) == KDA_OK);   // T < stride: no snapshot exists
}

void test_workspaces() {
    Prefill p(1, 256, 2, 128, 128, KDA_BF16);
    const size_t need =
        kda_chunk_fwd_chunk64_workspace_bytes(nullptr, 0, 1, 256, 2, 128, 128, KDA_BF16);
    EXPECT(need == kda::c64_mfma_workspace_bytes(4, 1, 2));
    EXPECT(kda_chunk_fwd_chunk64_workspace_bytes(nullptr, 0, 1, 256, 2, 128, 128, KDA_F32) == 0);
    EXPECT(kda_chunk_fwd_chunk64_workspace_bytes(nullptr, 0, 1, 256, 2, 120, 128, KDA_BF16) == 0);
    std::vector<unsigned char> ws(need + 256);
    unsigned char* al = ws.data() + (256 - reinterpret_cast<uintptr_t>(ws.data()) % 256) % 256;
    auto c64 = [&](void* w, size_t bytes) {
        reset();
        return kda_chunk_fwd_chunk64(p.q.data(), p.k.data(), p.v.data(), p.g.data(),
                                     p.beta.data(), p.h0.data(), nullptr, 0, p.o.data(),
                                     p.hT.data(), 1, 256, 2, 128, 128, KDA_BF16, w, bytes,
                                     nullptr);
    };
    EXPECT(c64(al, need) == KDA_OK && std::strcmp(g_last, "c64_mfma") == 0 && g_c64_chunks == 4);
    EXPECT(c64(al, need - 1) == KDA_ERR_WORKSPACE && g_launches == 0);
    EXPECT(c64(nullptr, need) == KDA_ERR_WORKSPACE && g_launches == 0);
    EXPECT(c64(al + 16, need) == KDA_ERR_WORKSPACE && g_launches == 0);

    // the split: one sequence of 4096 tokens and 2 heads plans several segments
    const int P = kda_chunk_fwd_split_segments(nullptr, 0, 0, 1, 4096, 2, 128, 128, KDA_BF16, 0);
    EXPECT(P > 1);
    EXPECT(kda_chunk_fwd_split_segments(nullptr, 0, 0, 1, 4096, 2, 128, 128, KDA_F32, 0) == 1);
    EXPECT(kda_chunk_fwd_split_segments(nullptr, 0, 0, 1, 4096, 2, 128, 128, KDA_BF16, 100) <= 16);
    const size_t sneed =
        kda_chunk_fwd_split_workspace_bytes(nullptr, 0, 0, 1, 4096, 2, 128, 128, KDA_BF16, 0);
    EXPECT(sneed > 0);
    Prefill s(1, 4096, 2, 128, 128, KDA_BF16);
    std::vector<unsigned char> sws(sneed + 256);
    unsigned char* sal = sws.data() + (256 - reinterpret_cast<uintptr_t>(sws.data()) % 256) % 256;
    auto split = [&](void* w, size_t bytes, int segs) {
        reset();
        return kda_chunk_fwd_split(s.q.data(), s.k.data(), s.v.data(), s.g.data(), s.beta.data(),
                                   s.h0.data(), nullptr, 0, 0, s.o.data(), s.hT.data(), 1, 4096, 2,
                                   128, 128, KDA_BF16, segs, w, bytes, nullptr);
    };
    EXPECT(split(sal, sneed, 0) == KDA_OK && g_launches == 2 && g_prefill.split == P);
    EXPECT(split(sal, sneed - 1, 0) == KDA_ERR_WORKSPACE && g_launches == 0);
    EXPECT(split(nullptr, 0, 1) == KDA_OK && g_launches == 1);   // one segment: no workspace
    EXPECT(split(sal, sneed, -1) == KDA_ERR_SHAPE && g_launches == 0);
}

void test_decode_and_stages() {
    const int N = 3, H = 2, d = 128;
    std::vector<uint16_t> q(N * H * d), k(N * H * d), v(N * H * d), g(N * H * d), b(N * H),
        o(N * H * d + 8), gate(N * H * d + 8), y(N * H * d + 8);
    std::vector<float> S(N * H * d * d + 4);
    auto dec = [&](float* s, void* out) {
        reset();
        return kda_decode_step(q.data(), k.data(), v.data(), g.data(), b.data(), s, out, N, H, d,
                               d, KDA_BF16, nullptr);
    };
    EXPECT(dec(S.data(), o.data()) == KDA_OK && std::strcmp(g_last, "decode_d128") == 0);
    // a state that is not 16-byte aligned takes the general path
    EXPECT(dec(S.data() + 1, o.data()) == KDA_OK && std::strcmp(g_last, "general") == 0);
    EXPECT(dec(nullptr, o.data()) == KDA_ERR_NULL && g_launches == 0);
    reset();
    EXPECT(kda_decode_step(q.data(), k.data(), v.data(), g.data(), b.data(), S.data(), o.data(),
                           0, H, d, d, KDA_BF16, nullptr) == KDA_OK && g_launches == 0);

    auto gated = [&](float eps, void* out, void* gt, void* yy) {
        reset();
        return kda_decode_step_gated(q.data(), k.data(), v.data(), g.data(), b.data(), S.data(),
                                     gt, nullptr, eps, out, yy, N, H, d, d, KDA_BF16, nullptr);
    };
    EXPECT(gated(1e-6f, o.data(), gate.data(), y.data()) == KDA_OK && g_launches == 1);
    EXPECT(gated(-1.f, o.data(), gate.data(), y.data()) == KDA_ERR_RANGE && g_launches == 0);
    EXPECT(gated(1e-6f, o.data(), nullptr, y.data()) == KDA_ERR_NULL && g_launches == 0);
    // 2-byte offsets: not even 8-byte aligned, so neither the fused kernel nor the output stage
    unsigned char* o2 = reinterpret_cast<unsigned char*>(o.data()) + 2;
    EXPECT(gated(1e-6f, o2, gate.data(), y.data()) == KDA_ERR_ALIGN && g_launches == 0);

    auto og = [&](float eps, const void* oo, int T) {
        reset();
        return kda_output_gate(oo, gate.data(), nullptr, eps, y.data(), T, H, d, KDA_BF16,
                               nullptr);
    };
    EXPECT(og(1e-6f, o.data(), N) == KDA_OK && g_launches == 1);
    EXPECT(og(1e-6f, o2, N) == KDA_ERR_ALIGN && g_launches == 0);
    EXPECT(og(-0.f, o.data(), N) == KDA_OK);
    EXPECT(og(__builtin_nanf(""), o.data(), N) == KDA_ERR_RANGE && g_launches == 0);
    EXPECT(og(__builtin_inff(), o.data(), N) == KDA_ERR_RANGE && g_launches == 0);
    EXPECT(og(1e-6f, nullptr, 0) == KDA_OK && g_launches == 0);
    EXPECT(og(1e-6f, o.data(), -1) == KDA_ERR_SHAPE);
}

void test_gated_prefill() {
    // fused: bf16, 128 x 128 heads, N * H >= 256 pairs -> one launch carrying the gate
    auto run = [&](Prefill& p, void* gate, void* y, bool with_o, float eps) {
        reset();
        return kda_chunk_fwd_gated(p.q.data(), p.k.data(), p.v.data(), p.g.data(), p.beta.data(),
                                   p.h0.data(), p.cup(), p.nseq(), gate, nullptr, eps,
                                   with_o ? p.o.data() : nullptr, y, p.hT.data(), p.B, p.T, p.H,
                                   p.dk, p.dv, p.dtype, nullptr);
    };
    {
        Prefill p(2, 32, 128, 128, 128, KDA_BF16);
        std::vector<unsigned char> gate(p.o.size()), y(p.o.size());
        EXPECT(kda_chunk_fwd_gated_fuses(0, 2, 128, 128, 128, KDA_BF16, 0) == 1);
        EXPECT(run(p, gate.data(), y.data(), false, 1e-6f) == KDA_OK);
        EXPECT(g_launches == 1 && std::strcmp(g_last, "mfma") == 0);
        EXPECT(g_prefill.gate == gate.data() && g_prefill.y == y.data() && g_prefill.o == nullptr);
        EXPECT(run(p, gate.data(), y.data(), false, -1.f) == KDA_ERR_RANGE && g_launches == 0);
        EXPECT(run(p, nullptr, y.data(), false, 1e-6f) == KDA_ERR_NULL && g_launches == 0);
        EXPECT(run(p, gate.data() + 2, y.data(), false, 1e-6f) == KDA_ERR_ALIGN &&
               g_launches == 0);
    }
    {
        // unfused (too few pairs): the prefill writes o into y, then the output stage in place
        Prefill p(1, 40, 2, 128, 128, KDA_BF16);
        std::vector<unsigned char> gate(p.o.size()), y(p.o.size());
        EXPECT(kda_chunk_fwd_gated_fuses(0, 1, 2, 128, 128, KDA_BF16, 0) == 0);
        EXPECT(run(p, gate.data(), y.data(), false, 1e-6f) == KDA_OK);
        EXPECT(g_launches == 2 && std::strcmp(g_last, "output_gate") == 0);
        EXPECT(g_prefill.o == y.data() && g_prefill.gate == nullptr);
        EXPECT(run(p, gate.data(), y.data(), true, 1e-6f) == KDA_OK && g_prefill.o == p.o.data());
    }
}

void test_frontend() {
    const int T = 20, H = 2, d = 64;
    std::vector<float> xq(T * H * d + 4), xk(T * H * d + 4), xv(T * H * d + 4), xz(T * H * d + 4),
        xb(T * H), wq(H * d * 4), wk(H * d * 4), wv(H * d * 4), zb(H * d), A(H),
        q(T * H * d + 4), k(T * H * d + 4), v(T * H * d + 4), g(T * H * d + 4), beta(T * H),
        cin(2 * 3 * H * 3 * d + 4), cout(2 * 3 * H * 3 * d + 4);
    auto fe = [&](float gmin, const int32_t* cu, int ns, int B, const void* xqp) {
        reset();
        return kda_frontend(xqp, xk.data(), xv.data(), xz.data(), xb.data(), wq.data(), wk.data(),
                            wv.data(), zb.data(), A.data(), gmin, 1e-6f, cu, ns, cin.data(),
                            cout.data(), q.data(), k.data(), v.data(), g.data(), beta.data(), B,
                            T, H, d, d, KDA_F32, nullptr);
    };
    EXPECT(fe(-5.f, nullptr, 0, 1, xq.data()) == KDA_OK && g_launches == 1);
    EXPECT(fe(0.f, nullptr, 0, 1, xq.data()) == KDA_ERR_RANGE && g_launches == 0);
    EXPECT(fe(-5.f, nullptr, 0, 1, nullptr) == KDA_ERR_NULL && g_launches == 0);
    EXPECT(fe(-5.f, nullptr, 0, 1, xq.data() + 1) == KDA_ERR_ALIGN && g_launches == 0);
    const std::vector<int32_t> cu = {0, 5, 20};
    EXPECT(fe(-5.f, cu.data(), 2, 1, xq.data()) == KDA_OK && g_launches == 1);
    EXPECT(fe(-5.f, cu.data(), 2, 2, xq.data()) == KDA_ERR_SEQLENS && g_launches == 0);
    set_validate(true);
    const std::vector<int32_t> bad = {0, 25, 20};
    EXPECT(fe(-5.f, bad.data(), 2, 1, xq.data()) == KDA_ERR_SEQLENS && g_launches == 0);
    set_validate(false);
}
void test_layer_decode() {
    const int N = 3, H = 2, d = 128;
    std::vector<uint16_t> xq(N * H * d), xk(N * H * d), xv(N * H * d), xz(N * H * d), xb(N * H),
        gate(N * H * d + 8), o(N * H * d + 8), y(N * H * d + 8), conv(N * 3 * H * 3 * d);
    std::vector<float> wq(H * d * 4), wk(H * d * 4), wv(H * d * 4), zb(H * d), A(H),
        S(N * H * d * d + 4);
    auto lay = [&](float gmin, float eps, void* cs, float* s, void* gt, void* oo, void* yy, int dk,
                   int n) {
        reset();
        return kda_decode_step_layer(xq.data(), xk.data(), xv.data(), xz.data(), xb.data(),
                                     wq.data(), wk.data(), wv.data(), zb.data(), A.data(), gmin,
                                     1e-6f, cs, s, gt, nullptr, eps, oo, yy, n, H, dk, dk,
                                     KDA_BF16, nullptr);
    };
    EXPECT(lay(-5.f, 1e-6f, conv.data(), S.data(), gate.data(), nullptr, y.data(), d, N) ==
               KDA_OK &&
           g_launches == 1 && std::strcmp(g_last, "decode_d128") == 0);
    // one launch carrying the input stage and the output stage; no q, k, v, g or beta buffers
    EXPECT(g_decode.xq == xq.data() && g_decode.xb == xb.data() && g_decode.conv == conv.data() &&
           g_decode.gate == gate.data() && g_decode.y == y.data() && g_decode.o == nullptr &&
           g_decode.q == nullptr && g_decode.beta == nullptr && g_decode.g_min == -5.f);
    EXPECT(lay(-5.f, 1e-6f, conv.data(), S.data(), gate.data(), o.data(), y.data(), d, N) ==
               KDA_OK && g_decode.o == o.data());
    EXPECT(lay(-5.f, 1e-6f, conv.data(), S.data(), gate.data(), nullptr, y.data(), 64, N) ==
               KDA_ERR_UNSUPPORTED && g_launches == 0);
    EXPECT(lay(0.f, 1e-6f, conv.data(), S.data(), gate.data(), nullptr, y.data(), d, N) ==
               KDA_ERR_RANGE && g_launches == 0);
    EXPECT(lay(-5.f, -1.f, conv.data(), S.data(), gate.data(), nullptr, y.data(), d, N) ==
               KDA_ERR_RANGE && g_launches == 0);
    EXPECT(lay(-5.f, 1e-6f, nullptr, S.data(), gate.data(), nullptr, y.data(), d, N) ==
               KDA_ERR_NULL && g_launches == 0);
    EXPECT(lay(-5.f, 1e-6f, conv.data(), S.data() + 1, gate.data(), nullptr, y.data(), d, N) ==
               KDA_ERR_ALIGN && g_launches == 0);
    unsigned char* y2 = reinterpret_cast<unsigned char*>(y.data()) + 2;
    EXPECT(lay(-5.f, 1e-6f, conv.data(), S.data(), gate.data(), nullptr, y2, d, N) ==
               KDA_ERR_ALIGN && g_launches == 0);
    EXPECT(lay(-5.f, 1e-6f, nullptr, nullptr, nullptr, nullptr, nullptr, d, 0) == KDA_OK &&
           g_launches == 0);
}
}  // namespace

int main() {
    unsetenv("KDA_VALIDATE");
    unsetenv("KDA_FORCE_GENERAL");
    test_status_strings();
    test_prefill_dispatch();
    test_prefill_rejects();
    test_validate_mode();
    test_snapshots_args();
    test_workspaces();
    test_decode_and_stages();
    test_gated_prefill();
    test_frontend();
    test_layer_decode();
    if (g_failures) {
        std::fprintf(stderr, "%d expectation(s) failed\n", g_failures);
        return 1;
    }
    std::printf("abi driver: all expectations hold\n");
    return 0;
}
