// The library driven through its C ABI alone: no Python, no PyTorch. Device buffers come
// from hipMalloc, work goes on one hipStream_t, and every result is checked on the host
// against properties and closed forms that need no reference implementation:
//   gate      ids distinct and in range, in descending logit order with ties to the lower
//             id, no unselected logit above a selected one; weights sum to 1;
//   layout    counts are the histogram of the ids; a placed route's slot is the number of
//             earlier tokens that chose its expert (the column cumsum minus one, counted by
//             brute force); a route is dropped exactly when that number reaches the
//             capacity; src inverts dst; offsets are the exclusive scan of the segments;
//   dispatch  every buffer row is its token's row bit for bit, unfilled rows are zero;
//   combine   with unit weights over integer-valued rows, token t comes back as exactly
//             (placed routes of t) * x[t]; the dispatch backward of the buffer likewise;
//   backward  grad_E[dst] is the float32 product w * grad_y; with the buffer as expert
//             output, grad_w[t,j] is exactly sum_m x[t,m]^2 (integers); the gate gradient
//             is zero off the selection and sums to zero over it (softmax Jacobian);
//   replay    byte-identical to the dispatch; a changed route sets the mismatch flag;
//   static    the layout built with its tile tables in the library's static scratch
//             array, in a workspace of the handle's share only, equals the other;
//   options, variants and the grouped expert GEMM: see run_variants_case;
//   errors    bad arguments return their status and a message, enqueueing nothing.
// Prints "c_abi_check: ok" and exits 0, or lists the failures and exits 1.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "moe_gate.h"

static int g_failures = 0;

#define CHECK(cond, ...)                                               \
  do {                                                                 \
    if (!(cond)) {                                                     \
      if (++g_failures <= 20) {                                        \
        std::fprintf(stderr, "FAIL line %d: ", __LINE__);              \
        std::fprintf(stderr, __VA_ARGS__);                             \
        std::fputc('\n', stderr);                                      \
      }                                                                \
    }                                                                  \
  } while (0)

#define HIP_OK(call)                                                                   \
  do {                                                                                 \
    const hipError_t e_ = (call);                                                      \
    if (e_ != hipSuccess) {                                                            \
      std::fprintf(stderr, "%s: %s (line %d)\n", #call, hipGetErrorString(e_), __LINE__); \
      std::exit(2);                                                                    \
    }                                                                                  \
  } while (0)

#define MOE_OK_(call)                                                                  \
  do {                                                                                 \
    const moe_status_t s_ = (call);                                                    \
    if (s_ != MOE_OK) {                                                                \
      std::fprintf(stderr, "%s: %s: %s (line %d)\n", #call, moe_status_string(s_),     \
                   moe_last_error(), __LINE__);                                        \
      std::exit(3);                                                                    \
    }                                                                                  \
  } while (0)

// A device array of n elements (at least one byte is allocated, so pointers are never
// NULL even for empty arrays).
template <class T>
struct Dev {
  T* p = nullptr;
  size_t n = 0;
  explicit Dev(size_t count) : n(count) { HIP_OK(hipMalloc(&p, std::max<size_t>(n, 1) * sizeof(T))); }
  ~Dev() { (void)hipFree(p); }
  Dev(const Dev&) = delete;
  Dev& operator=(const Dev&) = delete;
  void put(const std::vector<T>& h) {
    if (n) HIP_OK(hipMemcpy(p, h.data(), n * sizeof(T), hipMemcpyHostToDevice));
  }
  std::vector<T> get() const {
    std::vector<T> h(n);
    if (n) HIP_OK(hipMemcpy(h.data(), p, n * sizeof(T), hipMemcpyDeviceToHost));
    return h;
  }
};

// splitmix64: a small counter-based generator for the inputs
struct Rng {
  uint64_t state;
  uint64_t next() {
    uint64_t z = (state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
  }
  int below(int n) { return static_cast<int>(next() % static_cast<uint64_t>(n)); }
};

static bool same_bits(float a, float b) { return std::memcmp(&a, &b, sizeof(float)) == 0; }

static void run_case(int s, int e, int k, int m, int cap, uint64_t seed, hipStream_t st) {
  std::printf("case s=%d e=%d k=%d m=%d capacity=%d\n", s, e, k, m, cap);
  std::fflush(stdout);
  Rng rng{seed};
  // logits on a coarse grid (multiples of 1/8 in [-4, 4)) so that ties occur
  std::vector<float> logits(static_cast<size_t>(s) * e);
  for (auto& v : logits) v = static_cast<float>(rng.below(64) - 32) / 8.0f;
  // integer-valued rows: every sum below is exact in float32
  std::vector<float> x(static_cast<size_t>(s) * m);
  for (auto& v : x) v = static_cast<float>(rng.below(17) - 8);

  Dev<float> d_logits(logits.size()), d_x(x.size()), d_w(static_cast<size_t>(s) * k),
      d_ones(static_cast<size_t>(s) * k), d_y(x.size()), d_gx(x.size()),
      d_gw(static_cast<size_t>(s) * k), d_gl(static_cast<size_t>(s) * e);
  Dev<int32_t> d_idx(static_cast<size_t>(s) * k);
  d_logits.put(logits);
  d_x.put(x);
  d_ones.put(std::vector<float>(static_cast<size_t>(s) * k, 1.0f));

  // (1) gate
  MOE_OK_(moe_gate_topk(d_logits.p, s, e, k, d_idx.p, d_w.p, st));
  HIP_OK(hipStreamSynchronize(st));
  const std::vector<int32_t> idx = d_idx.get();
  const std::vector<float> w = d_w.get();
  for (int t = 0; t < s; ++t) {
    const float* l = &logits[static_cast<size_t>(t) * e];
    const int32_t* id = &idx[static_cast<size_t>(t) * k];
    std::vector<char> chosen(e, 0);
    double wsum = 0.0;
    for (int j = 0; j < k; ++j) {
      CHECK(id[j] >= 0 && id[j] < e, "t=%d j=%d id %d out of range", t, j, id[j]);
      if (id[j] < 0 || id[j] >= e) continue;
      CHECK(!chosen[id[j]], "t=%d expert %d chosen twice", t, id[j]);
      chosen[id[j]] = 1;
      if (j > 0 && id[j - 1] >= 0 && id[j - 1] < e) {
        const float a = l[id[j - 1]], b = l[id[j]];
        CHECK(a > b || (a == b && id[j - 1] < id[j]), "t=%d routes %d,%d out of order", t, j - 1, j);
        CHECK(w[static_cast<size_t>(t) * k + j - 1] >= w[static_cast<size_t>(t) * k + j],
              "t=%d weights not descending", t);
      }
      wsum += w[static_cast<size_t>(t) * k + j];
    }
    CHECK(std::fabs(wsum - 1.0) <= 1e-6, "t=%d weights sum to %.9f", t, wsum);
    const int last = id[k - 1];
    if (last >= 0 && last < e)
      for (int x2 = 0; x2 < e; ++x2)
        if (!chosen[x2])
          CHECK(l[x2] < l[last] || (l[x2] == l[last] && x2 > last),
                "t=%d unselected expert %d beats selected %d", t, x2, last);
  }

  // (2) layout
  const size_t ws_bytes = moe_layout_workspace_bytes(s, e, k, cap);
  CHECK(ws_bytes > 0, "workspace size 0");
  Dev<unsigned char> ws(ws_bytes);
  moe_layout_t L;
  MOE_OK_(moe_dispatch_layout(d_idx.p, s, e, k, cap, ws.p, ws_bytes, &L, st));
  const int64_t rows = L.rows;
  CHECK(rows == (cap > 0 ? static_cast<int64_t>(e) * cap : static_cast<int64_t>(s) * k),
        "rows %lld", static_cast<long long>(rows));
  std::vector<int32_t> counts(e), kept(e), offsets(e + 1), dst(static_cast<size_t>(s) * k),
      src(static_cast<size_t>(rows));
  HIP_OK(hipStreamSynchronize(st));
  HIP_OK(hipMemcpy(counts.data(), L.counts, sizeof(int32_t) * e, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(kept.data(), L.kept, sizeof(int32_t) * e, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(offsets.data(), L.offsets, sizeof(int32_t) * (e + 1), hipMemcpyDeviceToHost));
  if (!dst.empty())
    HIP_OK(hipMemcpy(dst.data(), L.dst, sizeof(int32_t) * dst.size(), hipMemcpyDeviceToHost));
  if (!src.empty())
    HIP_OK(hipMemcpy(src.data(), L.src, sizeof(int32_t) * src.size(), hipMemcpyDeviceToHost));
  int32_t flags = -1;
  MOE_OK_(moe_layout_read(&L, &flags, nullptr, st));
  CHECK(flags == 0, "flags %d on valid routing", flags);

  // the same layout with its tile tables in the library's static scratch array, in a
  // workspace of only the handle's share: the same arrays, flags and checksum
  {
    const size_t hb = MOE_LAYOUT_HANDLE_BYTES(s, e, k, rows);
    CHECK(hb <= ws_bytes, "handle share %zu above the workspace size %zu", hb, ws_bytes);
    Dev<unsigned char> ws2(hb);
    moe_layout_t L2;
    MOE_OK_(moe_dispatch_layout_static_scratch(d_idx.p, s, e, k, cap, nullptr, ws2.p, hb, &L2, st));
    CHECK(L2.rows == rows, "static-scratch layout rows %lld", static_cast<long long>(L2.rows));
    HIP_OK(hipStreamSynchronize(st));
    auto fetch = [](const int32_t* p, size_t n) {
      std::vector<int32_t> h(n);
      if (n) HIP_OK(hipMemcpy(h.data(), p, n * sizeof(int32_t), hipMemcpyDeviceToHost));
      return h;
    };
    CHECK(fetch(L2.counts, e) == counts && fetch(L2.kept, e) == kept && fetch(L2.offsets, e + 1) == offsets,
          "static-scratch layout: counts, kept or offsets differ");
    CHECK(fetch(L2.dst, dst.size()) == dst && fetch(L2.src, src.size()) == src,
          "static-scratch layout: dst or src differ");
    CHECK(fetch(L2.route_idx, idx.size()) == idx, "static-scratch layout: routing copy differs");
    int32_t f2 = -1;
    uint64_t c1 = 0, c2 = 1;
    MOE_OK_(moe_layout_read(&L, nullptr, &c1, st));
    MOE_OK_(moe_layout_read(&L2, &f2, &c2, st));
    CHECK(f2 == 0 && c1 == c2, "static-scratch layout: flags %d, checksum %llu vs %llu", f2,
          static_cast<unsigned long long>(c2), static_cast<unsigned long long>(c1));
  }

  std::vector<int32_t> seen(e, 0), placed_of_token(s, 0);
  std::vector<int> row_refs(static_cast<size_t>(rows), 0);
  int32_t expect_off = 0;
  for (int x2 = 0; x2 < e; ++x2) {
    CHECK(offsets[x2] == expect_off, "offsets[%d] = %d, want %d", x2, offsets[x2], expect_off);
    expect_off += cap > 0 ? cap : counts[x2];
  }
  CHECK(offsets[e] == (cap > 0 ? e * cap : s * k), "offsets[e] = %d", offsets[e]);
  for (int t = 0; t < s; ++t)
    for (int j = 0; j < k; ++j) {
      const int x2 = idx[static_cast<size_t>(t) * k + j];
      const int slot = seen[x2]++;  // earlier tokens that chose x2
      const int32_t d = dst[static_cast<size_t>(t) * k + j];
      if (cap > 0 && slot >= cap) {
        CHECK(d == -1, "t=%d j=%d slot %d past capacity but placed at %d", t, j, slot, d);
        continue;
      }
      CHECK(d == offsets[x2] + slot, "t=%d j=%d dst %d, want %d", t, j, d, offsets[x2] + slot);
      if (d >= 0 && d < rows) {
        ++row_refs[d];
        CHECK(src[d] == t, "src[%d] = %d, want %d", d, src[d], t);
      }
      ++placed_of_token[t];
    }
  for (int x2 = 0; x2 < e; ++x2) {
    CHECK(counts[x2] == seen[x2], "counts[%d] = %d, want %d", x2, counts[x2], seen[x2]);
    CHECK(kept[x2] == (cap > 0 ? std::min(seen[x2], cap) : seen[x2]), "kept[%d] = %d", x2, kept[x2]);
  }
  for (int64_t r = 0; r < rows; ++r)
    CHECK((row_refs[r] == 1) == (src[r] >= 0) && row_refs[r] <= 1, "row %lld referenced %d times, src %d",
          static_cast<long long>(r), row_refs[r], src[r]);

  // (3) dispatch, and its replay
  Dev<float> d_buf(static_cast<size_t>(rows) * m), d_rep(static_cast<size_t>(rows) * m),
      d_gE(static_cast<size_t>(rows) * m);
  MOE_OK_(moe_dispatch(&L, d_x.p, m, MOE_F32, d_buf.p, st));
  MOE_OK_(moe_dispatch_replay(&L, d_idx.p, d_x.p, m, MOE_F32, d_rep.p, st));
  HIP_OK(hipStreamSynchronize(st));
  const std::vector<float> buf = d_buf.get();
  const std::vector<float> rep = d_rep.get();
  for (int64_t r = 0; r < rows; ++r)
    for (int i = 0; i < m; ++i) {
      const float got = buf[static_cast<size_t>(r) * m + i];
      const float want = src[r] >= 0 ? x[static_cast<size_t>(src[r]) * m + i] : 0.0f;
      CHECK(same_bits(got, want), "buffer row %lld col %d: %g, want %g", static_cast<long long>(r), i, got, want);
    }
  CHECK(buf.empty() || std::memcmp(buf.data(), rep.data(), buf.size() * sizeof(float)) == 0,
        "replay differs from dispatch");
  MOE_OK_(moe_layout_read(&L, &flags, nullptr, st));
  CHECK(flags == 0, "flags %d after a faithful replay", flags);

  // (4) unit-weight combine and the dispatch backward of the buffer: kept_t * x[t]
  MOE_OK_(moe_combine(&L, d_buf.p, d_ones.p, m, MOE_F32, d_y.p, st));
  MOE_OK_(moe_dispatch_backward(&L, d_buf.p, m, MOE_F32, d_gx.p, st));
  HIP_OK(hipStreamSynchronize(st));
  const std::vector<float> y = d_y.get();
  const std::vector<float> gx = d_gx.get();
  for (int t = 0; t < s; ++t)
    for (int i = 0; i < m; ++i) {
      const float want = static_cast<float>(placed_of_token[t]) * x[static_cast<size_t>(t) * m + i];
      CHECK(y[static_cast<size_t>(t) * m + i] == want, "combine t=%d col %d: %g, want %g", t, i,
            y[static_cast<size_t>(t) * m + i], want);
      CHECK(gx[static_cast<size_t>(t) * m + i] == want, "dispatch backward t=%d col %d", t, i);
    }

  // (5) combine backward with grad_y = x over the buffer as expert output, and the gate
  // backward of the resulting weight gradient
  MOE_OK_(moe_combine_backward(&L, d_x.p, d_buf.p, d_w.p, m, MOE_F32, d_gE.p, d_gw.p, st));
  MOE_OK_(moe_gate_topk_backward(d_idx.p, d_w.p, d_gw.p, s, e, k, d_gl.p, st));
  HIP_OK(hipStreamSynchronize(st));
  const std::vector<float> gE = d_gE.get();
  const std::vector<float> gw = d_gw.get();
  const std::vector<float> gl = d_gl.get();
  for (int t = 0; t < s; ++t) {
    double sq = 0.0;
    for (int i = 0; i < m; ++i) sq += static_cast<double>(x[static_cast<size_t>(t) * m + i]) * x[static_cast<size_t>(t) * m + i];
    double gsum = 0.0, gabs = 0.0;
    for (int j = 0; j < k; ++j) {
      const size_t o = static_cast<size_t>(t) * k + j;
      const int32_t d = dst[o];
      CHECK(gw[o] == (d >= 0 ? static_cast<float>(sq) : 0.0f), "grad_w t=%d j=%d: %g, want %g", t, j, gw[o],
            d >= 0 ? sq : 0.0);
      if (d >= 0)
        for (int i = 0; i < m; ++i) {
          const float want = w[o] * x[static_cast<size_t>(t) * m + i];  // one float32 product
          CHECK(same_bits(gE[static_cast<size_t>(d) * m + i], want), "grad_E row %d col %d", d, i);
        }
      const float g = gl[static_cast<size_t>(t) * e + idx[o]];
      gsum += g;
      gabs += std::fabs(static_cast<double>(w[o]) * gw[o]);
    }
    CHECK(std::fabs(gsum) <= 1e-6 * gabs + 1e-30, "t=%d gate gradient sums to %g over the selection", t, gsum);
    std::vector<char> chosen(e, 0);
    for (int j = 0; j < k; ++j) chosen[idx[static_cast<size_t>(t) * k + j]] = 1;
    for (int x2 = 0; x2 < e; ++x2)
      if (!chosen[x2]) CHECK(gl[static_cast<size_t>(t) * e + x2] == 0.0f, "t=%d gate gradient off the selection", t);
  }
  for (int64_t r = 0; r < rows; ++r)
    if (src[r] < 0)
      for (int i = 0; i < m; ++i) CHECK(gE[static_cast<size_t>(r) * m + i] == 0.0f, "grad_E unfilled row %lld", static_cast<long long>(r));

  // replay against changed routing: the copy still follows the layout, the flag is set
  if (s > 0 && k < e) {
    std::vector<int32_t> idx2 = idx;
    for (int x2 = 0; x2 < e; ++x2)
      if (std::find(idx2.begin(), idx2.begin() + k, x2) == idx2.begin() + k) {
        idx2[0] = x2;
        break;
      }
    Dev<int32_t> d_idx2(idx2.size());
    d_idx2.put(idx2);
    MOE_OK_(moe_dispatch_replay(&L, d_idx2.p, d_x.p, m, MOE_F32, d_rep.p, st));
    MOE_OK_(moe_layout_read(&L, &flags, nullptr, st));
    CHECK((flags & MOE_FLAG_REPLAY_MISMATCH) != 0, "changed routing not flagged (flags %d)", flags);
    const std::vector<float> rep2 = d_rep.get();
    CHECK(std::memcmp(buf.data(), rep2.data(), buf.size() * sizeof(float)) == 0, "flagged replay differs");
  }
}

static uint16_t bf16_of(float v) {  // exact for the small integers used here
  uint32_t u;
  std::memcpy(&u, &v, sizeof(u));
  return static_cast<uint16_t>(u >> 16);
}

static float float_of_bf16(uint16_t h) {
  const uint32_t u = static_cast<uint32_t>(h) << 16;
  float v;
  std::memcpy(&v, &u, sizeof(v));
  return v;
}

static std::vector<int32_t> read_i32(const int32_t* p, size_t n) {
  std::vector<int32_t> h(n);
  if (n) HIP_OK(hipMemcpy(h.data(), p, n * sizeof(int32_t), hipMemcpyDeviceToHost));
  return h;
}

// The layout options, the variants and the grouped expert GEMM through the ABI:
//   pad_multiple  segments rounded up to the multiple, pad rows never referenced;
//   route_major   with a capacity, a route's slot counts the earlier routes of lower rank
//                 j' < j (any token) and of the same rank from earlier tokens;
//   weighted dispatch out[dst] = w * x (one float32 product), its unweighted combine and
//                 its backward, with power-of-two weights over integer rows (exact sums);
//   renormalisation the kept weights of a token sum to one, and the backward of a
//                 gradient along the weights themselves is zero;
//   expert GEMM   forward (gathered and on the dispatched buffer, with and without route
//                 weights), input-row and weight gradients: small-integer bf16 operands,
//                 so every sum is an exact integer.
static void run_variants_case(hipStream_t st) {
  const int s = 200, e = 12, k = 3, m = 64, n = 32, cap = 40;
  std::printf("case variants and expert GEMM s=%d e=%d k=%d m=%d n=%d\n", s, e, k, m, n);
  std::fflush(stdout);
  Rng rng{77};
  std::vector<int32_t> idx(static_cast<size_t>(s) * k);
  for (int t = 0; t < s; ++t) {  // k distinct experts per token
    for (int j = 0; j < k; ++j) {
      int x;
      bool again;
      do {
        x = rng.below(e);
        again = false;
        for (int q = 0; q < j; ++q) again |= idx[static_cast<size_t>(t) * k + q] == x;
      } while (again);
      idx[static_cast<size_t>(t) * k + j] = x;
    }
  }
  const float wchoice[4] = {0.25f, 0.5f, 1.0f, 2.0f};
  std::vector<float> w(static_cast<size_t>(s) * k), x(static_cast<size_t>(s) * m);
  for (auto& v : w) v = wchoice[rng.below(4)];
  for (auto& v : x) v = static_cast<float>(rng.below(3) - 1);  // -1, 0, 1
  Dev<int32_t> d_idx(idx.size());
  Dev<float> d_w(w.size()), d_x(x.size());
  d_idx.put(idx);
  d_w.put(w);
  d_x.put(x);

  // pad_multiple = 8, dropless
  {
    moe_layout_options_t o{0, 8};
    const size_t wsb = moe_layout_workspace_bytes_ex(s, e, k, 0, &o);
    Dev<unsigned char> ws(wsb);
    moe_layout_t L;
    MOE_OK_(moe_dispatch_layout_ex(d_idx.p, s, e, k, 0, &o, ws.p, wsb, &L, st));
    HIP_OK(hipStreamSynchronize(st));
    CHECK(L.rows == static_cast<int64_t>(s) * k + e * 7, "padded rows %lld", static_cast<long long>(L.rows));
    const auto offsets = read_i32(L.offsets, e + 1);
    const auto dst = read_i32(L.dst, idx.size());
    const auto src = read_i32(L.src, static_cast<size_t>(L.rows));
    std::vector<int> seen(e, 0);
    for (int t = 0; t < s; ++t)
      for (int j = 0; j < k; ++j) {
        const int xe = idx[static_cast<size_t>(t) * k + j];
        const int d = dst[static_cast<size_t>(t) * k + j];
        CHECK(d == offsets[xe] + seen[xe], "padded dst t=%d j=%d", t, j);
        if (d >= 0 && d < L.rows) CHECK(src[d] == t, "padded src");
        ++seen[xe];
      }
    int32_t off = 0;
    for (int xe = 0; xe < e; ++xe) {
      CHECK(offsets[xe] == off && off % 8 == 0, "padded offsets[%d]", xe);
      for (int32_t r = off + seen[xe]; r < off + (seen[xe] + 7) / 8 * 8; ++r) CHECK(src[r] == -1, "pad row %d", r);
      off += (seen[xe] + 7) / 8 * 8;
    }
  }

  // route-major slots with a capacity
  {
    moe_layout_options_t o{1, 1};
    const size_t wsb = moe_layout_workspace_bytes_ex(s, e, k, cap, &o);
    Dev<unsigned char> ws(wsb);
    moe_layout_t L;
    MOE_OK_(moe_dispatch_layout_ex(d_idx.p, s, e, k, cap, &o, ws.p, wsb, &L, st));
    HIP_OK(hipStreamSynchronize(st));
    const auto dst = read_i32(L.dst, idx.size());
    std::vector<int> seen(e, 0);
    for (int j = 0; j < k; ++j)
      for (int t = 0; t < s; ++t) {
        const int xe = idx[static_cast<size_t>(t) * k + j];
        const int slot = seen[xe]++;
        const int want = slot < cap ? xe * cap + slot : -1;
        CHECK(dst[static_cast<size_t>(t) * k + j] == want, "route-major dst t=%d j=%d: %d, want %d", t, j,
              dst[static_cast<size_t>(t) * k + j], want);
      }
  }

  // capacity layout for the weighted dispatch, renormalisation and the GEMMs
  const size_t wsb = moe_layout_workspace_bytes(s, e, k, cap);
  Dev<unsigned char> ws(wsb);
  moe_layout_t L;
  MOE_OK_(moe_dispatch_layout(d_idx.p, s, e, k, cap, ws.p, wsb, &L, st));
  HIP_OK(hipStreamSynchronize(st));
  const int64_t rows = L.rows;
  const auto dst = read_i32(L.dst, idx.size());
  const auto src = read_i32(L.src, static_cast<size_t>(rows));

  Dev<float> d_out(static_cast<size_t>(rows) * m), d_y(x.size()), d_gx(x.size()), d_gw(w.size());
  MOE_OK_(moe_dispatch_weighted(&L, d_x.p, d_w.p, m, MOE_F32, d_out.p, st));
  MOE_OK_(moe_combine(&L, d_out.p, nullptr, m, MOE_F32, d_y.p, st));
  MOE_OK_(moe_dispatch_weighted_backward(&L, d_out.p, d_x.p, d_w.p, m, MOE_F32, d_gx.p, d_gw.p, st));
  HIP_OK(hipStreamSynchronize(st));
  const auto out = d_out.get();
  const auto y = d_y.get();
  const auto gx = d_gx.get();
  const auto gw = d_gw.get();
  for (int t = 0; t < s; ++t) {
    float sw = 0.0f, sw2 = 0.0f, sq = 0.0f;
    for (int i = 0; i < m; ++i) sq += x[static_cast<size_t>(t) * m + i] * x[static_cast<size_t>(t) * m + i];
    for (int j = 0; j < k; ++j) {
      const size_t o = static_cast<size_t>(t) * k + j;
      if (dst[o] < 0) {
        CHECK(gw[o] == 0.0f, "weighted dispatch grad_w of a dropped route");
        continue;
      }
      sw += w[o];
      sw2 += w[o] * w[o];
      for (int i = 0; i < m; ++i)
        CHECK(same_bits(out[static_cast<size_t>(dst[o]) * m + i], w[o] * x[static_cast<size_t>(t) * m + i]),
              "weighted dispatch row %d", dst[o]);
      CHECK(gw[o] == w[o] * sq, "weighted dispatch grad_w t=%d j=%d", t, j);
    }
    for (int i = 0; i < m; ++i) {
      const float xv = x[static_cast<size_t>(t) * m + i];
      CHECK(y[static_cast<size_t>(t) * m + i] == sw * xv, "unweighted combine t=%d", t);
      CHECK(gx[static_cast<size_t>(t) * m + i] == sw2 * xv, "weighted dispatch grad_x t=%d", t);
    }
  }
  for (int64_t r = 0; r < rows; ++r)
    if (src[r] < 0)
      for (int i = 0; i < m; ++i) CHECK(out[static_cast<size_t>(r) * m + i] == 0.0f, "unfilled weighted row");

  // renormalisation over kept routes
  Dev<float> d_wr(w.size()), d_g(w.size()), d_gr(w.size());
  std::vector<float> g(w.size());
  for (size_t o = 0; o < g.size(); ++o) g[o] = w[o];  // a gradient along the weights
  d_g.put(g);
  MOE_OK_(moe_renormalize_kept(&L, d_w.p, d_wr.p, st));
  MOE_OK_(moe_renormalize_kept_backward(&L, d_w.p, d_g.p, d_gr.p, st));
  HIP_OK(hipStreamSynchronize(st));
  const auto wr = d_wr.get();
  const auto gr = d_gr.get();
  for (int t = 0; t < s; ++t) {
    double sum = 0.0, dotw = 0.0, mag = 0.0;
    int kept = 0;
    for (int j = 0; j < k; ++j) {
      const size_t o = static_cast<size_t>(t) * k + j;
      if (dst[o] < 0) {
        CHECK(wr[o] == 0.0f && gr[o] == 0.0f, "renormalised dropped route t=%d", t);
        continue;
      }
      ++kept;
      sum += wr[o];
      dotw += static_cast<double>(w[o]) * gr[o];
      mag += std::fabs(static_cast<double>(w[o]) * gr[o]) + std::fabs(static_cast<double>(g[o]));
    }
    if (kept) {
      CHECK(std::fabs(sum - 1.0) <= 1e-6, "renormalised weights of t=%d sum to %.9f", t, sum);
      CHECK(std::fabs(dotw) <= 1e-6 * mag + 1e-30, "renormalisation backward along w: %g", dotw);
    }
  }

  // grouped expert GEMM, bf16 small-integer operands
  std::vector<uint16_t> xb(x.size()), wb(static_cast<size_t>(e) * n * m), gb(static_cast<size_t>(rows) * n);
  for (size_t i = 0; i < x.size(); ++i) xb[i] = bf16_of(x[i]);
  for (auto& v : wb) v = bf16_of(static_cast<float>(rng.below(3) - 1));
  for (auto& v : gb) v = bf16_of(static_cast<float>(rng.below(3) - 1));
  Dev<uint16_t> d_xb(xb.size()), d_wb(wb.size()), d_gb(gb.size()), d_buf(static_cast<size_t>(rows) * m),
      d_h(static_cast<size_t>(rows) * n), d_h2(static_cast<size_t>(rows) * n), d_hs(static_cast<size_t>(rows) * n),
      d_ga(static_cast<size_t>(rows) * m), d_gwn(wb.size());
  Dev<float> d_gwf(wb.size());
  d_xb.put(xb);
  d_wb.put(wb);
  d_gb.put(gb);
  MOE_OK_(moe_dispatch(&L, d_xb.p, m, MOE_BF16, d_buf.p, st));
  MOE_OK_(moe_expert_gemm(&L, d_xb.p, 1, d_wb.p, m, n, MOE_BF16, nullptr, d_h.p, st));
  MOE_OK_(moe_expert_gemm(&L, d_buf.p, 0, d_wb.p, m, n, MOE_BF16, nullptr, d_h2.p, st));
  MOE_OK_(moe_expert_gemm(&L, d_xb.p, 1, d_wb.p, m, n, MOE_BF16, d_w.p, d_hs.p, st));
  MOE_OK_(moe_expert_gemm_dgrad(&L, d_gb.p, d_wb.p, m, n, MOE_BF16, d_ga.p, st));
  MOE_OK_(moe_expert_gemm_wgrad(&L, d_xb.p, 1, d_gb.p, m, n, MOE_BF16, MOE_F32, d_gwf.p, st));
  MOE_OK_(moe_expert_gemm_wgrad(&L, d_xb.p, 1, d_gb.p, m, n, MOE_BF16, MOE_BF16, d_gwn.p, st));
  HIP_OK(hipStreamSynchronize(st));
  const auto h = d_h.get(), h2 = d_h2.get(), hs = d_hs.get(), ga = d_ga.get(), gwn = d_gwn.get();
  const auto gwf = d_gwf.get();
  CHECK(h == h2, "gathered and buffered expert GEMM differ");
  std::vector<float> rw(static_cast<size_t>(rows), 0.0f);  // the route weight placed at each row
  for (size_t o = 0; o < dst.size(); ++o)
    if (dst[o] >= 0) rw[dst[o]] = w[o];
  std::vector<double> gwx(wb.size(), 0.0);
  for (int64_t r = 0; r < rows; ++r) {
    const int xe = static_cast<int>(r / cap);
    const bool filled = src[r] >= 0;
    for (int c = 0; c < n; ++c) {
      double acc = 0.0;
      if (filled)
        for (int i = 0; i < m; ++i)
          acc += static_cast<double>(x[static_cast<size_t>(src[r]) * m + i]) *
                 float_of_bf16(wb[(static_cast<size_t>(xe) * n + c) * m + i]);
      const size_t o = static_cast<size_t>(r) * n + c;
      CHECK(float_of_bf16(h[o]) == acc, "expert GEMM row %lld col %d", static_cast<long long>(r), c);
      CHECK(float_of_bf16(hs[o]) == rw[r] * acc, "scaled expert GEMM row %lld col %d", static_cast<long long>(r), c);
    }
    for (int i = 0; i < m; ++i) {
      double acc = 0.0;
      if (filled)
        for (int c = 0; c < n; ++c)
          acc += static_cast<double>(float_of_bf16(gb[static_cast<size_t>(r) * n + c])) *
                 float_of_bf16(wb[(static_cast<size_t>(xe) * n + c) * m + i]);
      CHECK(float_of_bf16(ga[static_cast<size_t>(r) * m + i]) == acc, "input-row gradient row %lld", static_cast<long long>(r));
    }
    if (filled)
      for (int c = 0; c < n; ++c)
        for (int i = 0; i < m; ++i)
          gwx[(static_cast<size_t>(xe) * n + c) * m + i] +=
              static_cast<double>(float_of_bf16(gb[static_cast<size_t>(r) * n + c])) * x[static_cast<size_t>(src[r]) * m + i];
  }
  for (size_t i = 0; i < gwx.size(); ++i) {
    CHECK(gwf[i] == gwx[i], "weight gradient (float32) element %zu", i);
    CHECK(float_of_bf16(gwn[i]) == gwx[i], "weight gradient (bf16) element %zu", i);
  }
}

static void check_errors(hipStream_t st) {
  std::printf("case argument errors\n");
  std::fflush(stdout);
  Dev<float> d_logits(64), d_w(8), d_x(64);
  Dev<int32_t> d_idx(8);
  CHECK(moe_gate_topk(d_logits.p, 8, 8, 9, d_idx.p, d_w.p, st) == MOE_ERR_INVALID_ARG, "k > e accepted");
  CHECK(std::strlen(moe_last_error()) > 0, "no message for k > e");
  CHECK(moe_gate_topk(nullptr, 8, 8, 1, d_idx.p, d_w.p, st) == MOE_ERR_INVALID_ARG, "NULL logits accepted");
  const size_t ws_bytes = moe_layout_workspace_bytes(8, 8, 1, 0);
  Dev<unsigned char> ws(ws_bytes);
  moe_layout_t L;
  CHECK(moe_dispatch_layout(d_idx.p, 8, 8, 1, 0, ws.p, ws_bytes - 1, &L, st) == MOE_ERR_WORKSPACE,
        "short workspace accepted");
  std::vector<int32_t> idx(8);
  for (int t = 0; t < 8; ++t) idx[t] = t;
  d_idx.put(idx);
  MOE_OK_(moe_dispatch_layout(d_idx.p, 8, 8, 1, 0, ws.p, ws_bytes, &L, st));
  Dev<float> d_out(64);
  // rows of 3 float32 are 12 bytes: not a multiple of 16
  CHECK(moe_dispatch(&L, d_x.p, 3, MOE_F32, d_out.p, st) == MOE_ERR_MISALIGNED, "12-byte rows accepted");
  moe_layout_t bad = L;
  bad.magic ^= 1u;
  CHECK(moe_dispatch(&bad, d_x.p, 8, MOE_F32, d_out.p, st) == MOE_ERR_HANDLE_MISMATCH, "foreign handle accepted");
  HIP_OK(hipStreamSynchronize(st));
}

int main() {
  std::printf("c_abi_check: library ABI version %d (header %d)\n", moe_abi_version(), MOE_ABI_VERSION);
  if (moe_abi_version() != MOE_ABI_VERSION) {
    std::fprintf(stderr, "library and header ABI versions differ\n");
    return 1;
  }
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  run_case(300, 16, 4, 40, 0, 1, st);      // dropless, ragged against every tile size
  run_case(300, 16, 4, 40, 60, 2, st);     // capacity drop
  run_case(1000, 64, 8, 64, 0, 3, st);
  run_case(97, 8, 2, 8, 5, 4, st);         // heavy drop, 32-byte rows
  run_case(513, 128, 16, 1028, 0, 5, st);  // rows of more than one 1 KiB group
  run_case(0, 8, 2, 16, 4, 6, st);         // empty batch: the buffer is all padding
  run_variants_case(st);
  check_errors(st);
  HIP_OK(hipStreamDestroy(st));
  if (g_failures != 0) {
    std::fprintf(stderr, "c_abi_check: %d failed checks\n", g_failures);
    return 1;
  }
  std::printf("c_abi_check: ok\n");
  return 0;
}
