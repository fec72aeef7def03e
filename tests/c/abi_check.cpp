// abi_check.cpp -- uses the library through its C ABI alone (include/grpo_rows.h,
// hipMalloc'd buffers, no PyTorch) and checks what holds by construction:
// status codes, finite outputs, 0 <= entropy <= log V, logp <= 0, dlogits rows
// summing to 0, all-zero rows exactly where zero_row says so (zero-advantage
// sequence without a reference model, masked tokens), the single pass agreeing
// with the two-pass forward + backward, the selective log-softmax and entropy
// ops agreeing with the GRPO forward, the selective log-softmax backward's row
// sums and zero rows, the fused-linear chunk's exact accumulation over two
// calls, and the small helpers' closed forms.
// Built by build() as tests/c/abi_check; run by tests/test_c_abi_gpu.py.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "grpo_rows.h"

static int failures = 0;
#define CHECK(cond, ...)                             \
  do {                                               \
    if (!(cond)) {                                   \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);             \
      std::fprintf(stderr, "\n");                    \
      ++failures;                                    \
    }                                                \
  } while (0)
#define HIP(x) CHECK((x) == hipSuccess, "%s", #x)
#define OK(x) do { const int st_ = (x); CHECK(st_ == GRPO_OK, "%s -> %s", #x, grpo_status_string(st_)); } while (0)

static uint32_t lcg(uint64_t& s) {
  s = s * 6364136223846793005ull + 1442695040888963407ull;
  return uint32_t(s >> 33);
}
static float unif(uint64_t& s, float lo, float hi) {
  return lo + (hi - lo) * float(lcg(s) & 0xFFFFFF) / float(0x1000000);
}
static uint16_t to_bf16(float f) {  // round to nearest even
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}
static float from_bf16(uint16_t b) {
  const uint32_t u = uint32_t(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

template <typename T>
static T* dalloc(size_t n) {
  void* p = nullptr;
  HIP(hipMalloc(&p, n * sizeof(T) + 16));
  return static_cast<T*>(p);
}
template <typename T>
static T* upload(const std::vector<T>& h) {
  T* d = dalloc<T>(h.size());
  HIP(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
  return d;
}
template <typename T>
static std::vector<T> download(const T* d, size_t n) {
  std::vector<T> h(n);
  HIP(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
  return h;
}

// One GRPO batch in `dtype` (GRPO_F32 or GRPO_BF16); logits values are the
// same up to the bf16 rounding.
static void run_case(int dtype, int64_t B, int64_t L, int64_t V, float T) {
  const int64_t N = B * L;
  const size_t es = dtype == GRPO_BF16 ? 2 : 4;
  // a row of dlogits sums to 0 up to the rounding of its elements
  const double rel = dtype == GRPO_BF16 ? 1.0 / 256.0 : 1e-5;
  uint64_t seed = 12345 + uint64_t(V);
  std::vector<float> zf(size_t(N * V));
  for (auto& x : zf) x = unif(seed, -4.0f, 4.0f);
  std::vector<uint16_t> zb(zf.size());
  if (dtype == GRPO_BF16)
    for (size_t i = 0; i < zf.size(); ++i) {
      zb[i] = to_bf16(zf[i]);
      zf[i] = from_bf16(zb[i]);
    }
  std::vector<int64_t> ids(N);
  for (auto& y : ids) y = int64_t(lcg(seed) % uint32_t(V));
  std::vector<float> old(N), adv(B);
  for (auto& o : old) o = -std::log(float(V)) + unif(seed, -0.5f, 0.5f);
  for (int64_t b = 0; b < B; ++b) adv[b] = b == 1 ? 0.0f : (b % 2 ? -0.5f : 0.7f);
  std::vector<uint8_t> mask(N, 1);
  for (int64_t t = L - 5; t < L; ++t) mask[(B - 1) * L + t] = 0;

  void* dz_in = dtype == GRPO_BF16 ? static_cast<void*>(upload(zb)) : static_cast<void*>(upload(zf));
  int64_t* d_ids = upload(ids);
  float* d_old = upload(old);
  float* d_adv = upload(adv);
  uint8_t* d_mask = upload(mask);
  float* d_w = dalloc<float>(N);
  OK(grpo_loss_weights(d_mask, B, L, GRPO_REDUCE_TOKEN, d_w, nullptr));
  float *d_loss = dalloc<float>(N), *d_logp = dalloc<float>(N), *d_lse = dalloc<float>(N),
        *d_H = dalloc<float>(N);
  uint8_t *d_clip = dalloc<uint8_t>(N), *d_zero = dalloc<uint8_t>(N);
  void* d_dl = dalloc<uint8_t>(size_t(N * V) * es);
  grpo_params p = {T, 0.04f, 0.2f, 0.28f, GRPO_TOKEN, 0};

  // two passes
  OK(grpo_logits_fwd(dz_in, dtype, B, L, V, V, d_ids, d_old, nullptr, d_adv, d_mask, &p, d_loss,
                     d_logp, d_lse, d_H, nullptr, d_clip, nullptr, nullptr, nullptr, nullptr));
  OK(grpo_logits_bwd(dz_in, dtype, B, L, V, V, d_ids, d_old, nullptr, d_adv, d_mask, &p, d_logp,
                     d_lse, nullptr, d_w, d_dl, V, d_zero, nullptr));
  HIP(hipDeviceSynchronize());
  const auto loss = download(d_loss, N), logp = download(d_logp, N), lse = download(d_lse, N),
             H = download(d_H, N), w = download(d_w, N);
  const auto zero = download(d_zero, N);
  std::vector<float> dl(size_t(N * V));
  if (dtype == GRPO_BF16) {
    const auto raw = download(static_cast<uint16_t*>(d_dl), size_t(N * V));
    for (size_t i = 0; i < raw.size(); ++i) dl[i] = from_bf16(raw[i]);
  } else {
    dl = download(static_cast<float*>(d_dl), size_t(N * V));
  }
  double wsum = 0.0;
  for (int64_t r = 0; r < N; ++r) {
    wsum += w[r];
    float zmax = -INFINITY;
    for (int64_t j = 0; j < V; ++j) zmax = std::fmax(zmax, zf[size_t(r * V + j)]);
    CHECK(std::isfinite(loss[r]) && std::isfinite(logp[r]) && std::isfinite(lse[r]), "row %ld finite", long(r));
    CHECK(logp[r] <= 1e-6f, "logp <= 0 (row %ld: %g)", long(r), logp[r]);
    CHECK(H[r] >= -1e-5f && H[r] <= std::log(float(V)) + 1e-4f, "0 <= H <= log V (row %ld: %g)", long(r), H[r]);
    CHECK(lse[r] >= zmax / T - 1e-4f, "lse >= max z / T (row %ld)", long(r));
    const bool must_zero = (r / L == 1) || mask[r] == 0;  // A = 0 without reference; masked
    if (must_zero) CHECK(zero[r] == 1, "zero_row set on row %ld", long(r));
    double s = 0.0, sa = 0.0;
    bool allzero = true;
    for (int64_t j = 0; j < V; ++j) {
      const float d = dl[size_t(r * V + j)];
      CHECK(std::isfinite(d), "dlogits finite");
      s += d;
      sa += std::fabs(d);
      if (d != 0.0f) allzero = false;
    }
    if (zero[r]) CHECK(allzero, "zero row %ld is all zeros", long(r));
    else CHECK(std::fabs(s) <= rel * sa + 1e-6, "row %ld sums to 0 (%g, sum |d| %g)", long(r), s, sa);
  }
  CHECK(std::fabs(wsum - 1.0) <= 1e-5, "token-mean weights sum to 1 (%g)", wsum);

  // single pass: same per-token outputs and dlogits up to rounding order
  if (int64_t(es) * V <= 131072) {
    float *d_loss1 = dalloc<float>(N), *d_logp1 = dalloc<float>(N), *d_lse1 = dalloc<float>(N);
    void* d_dl1 = dalloc<uint8_t>(size_t(N * V) * es);
    OK(grpo_logits_fwd_bwd(dz_in, dtype, B, L, V, V, d_ids, d_old, nullptr, d_adv, d_mask, &p,
                           d_w, d_loss1, d_logp1, d_lse1, nullptr, nullptr, nullptr, d_dl1, V,
                           nullptr, nullptr, nullptr));
    HIP(hipDeviceSynchronize());
    const auto loss1 = download(d_loss1, N), logp1 = download(d_logp1, N);
    for (int64_t r = 0; r < N; ++r) {
      CHECK(std::fabs(loss1[r] - loss[r]) <= 1e-5f * std::fabs(loss[r]) + 1e-6f, "single-pass loss row %ld", long(r));
      CHECK(std::fabs(logp1[r] - logp[r]) <= 1e-5f * std::fabs(logp[r]) + 1e-6f, "single-pass logp row %ld", long(r));
    }
    HIP(hipFree(d_loss1));
    HIP(hipFree(d_logp1));
    HIP(hipFree(d_lse1));
    HIP(hipFree(d_dl1));
  }

  // the axolotl-style ops agree with the GRPO forward at the same T
  float *d_lp2 = dalloc<float>(N), *d_lse2 = dalloc<float>(N), *d_H2 = dalloc<float>(N);
  OK(selective_log_softmax(dz_in, dtype, N, V, V, d_ids, T, d_lp2, d_lse2, nullptr));
  OK(entropy_from_logits(dz_in, dtype, N, V, V, T, d_H2, nullptr));
  // entropy backward with a zero upstream gradient on even rows
  std::vector<float> gH(N);
  for (int64_t r = 0; r < N; ++r) gH[r] = r % 2 ? 0.25f : 0.0f;
  float* d_gH = upload(gH);
  OK(entropy_from_logits_bwd(dz_in, dtype, N, V, V, T, d_lse, d_H, d_gH, d_dl, V, nullptr));
  HIP(hipDeviceSynchronize());
  const auto lp2 = download(d_lp2, N), H2 = download(d_H2, N);
  for (int64_t r = 0; r < N; ++r) {
    CHECK(std::fabs(lp2[r] - logp[r]) <= 1e-5f * std::fabs(logp[r]) + 1e-6f, "selective logp row %ld", long(r));
    CHECK(std::fabs(H2[r] - H[r]) <= 1e-5f * std::fabs(H[r]) + 1e-6f, "entropy row %ld", long(r));
  }
  std::vector<float> dh(size_t(N * V));
  if (dtype == GRPO_BF16) {
    const auto raw = download(static_cast<uint16_t*>(d_dl), size_t(N * V));
    for (size_t i = 0; i < raw.size(); ++i) dh[i] = from_bf16(raw[i]);
  } else {
    dh = download(static_cast<float*>(d_dl), size_t(N * V));
  }
  for (int64_t r = 0; r < N; ++r) {
    double s = 0.0, sa = 0.0;
    bool allzero = true;
    for (int64_t j = 0; j < V; ++j) {
      const float d = dh[size_t(r * V + j)];
      s += d;
      sa += std::fabs(d);
      if (d != 0.0f) allzero = false;
    }
    if (gH[r] == 0.0f) CHECK(allzero, "entropy backward zero row %ld", long(r));
    else CHECK(std::fabs(s) <= rel * sa + 1e-6, "entropy backward row %ld sums to 0", long(r));
  }

  // selective log-softmax backward with the same upstream pattern: rows sum
  // to 0, and a zero upstream gradient gives an all-zero row
  OK(selective_log_softmax_bwd(dz_in, dtype, N, V, V, d_ids, T, d_lse2, d_gH, d_dl, V, nullptr));
  HIP(hipDeviceSynchronize());
  std::vector<float> ds(size_t(N * V));
  if (dtype == GRPO_BF16) {
    const auto raw = download(static_cast<uint16_t*>(d_dl), size_t(N * V));
    for (size_t i = 0; i < raw.size(); ++i) ds[i] = from_bf16(raw[i]);
  } else {
    ds = download(static_cast<float*>(d_dl), size_t(N * V));
  }
  for (int64_t r = 0; r < N; ++r) {
    double s = 0.0, sa = 0.0;
    bool allzero = true;
    for (int64_t j = 0; j < V; ++j) {
      const float d = ds[size_t(r * V + j)];
      s += d;
      sa += std::fabs(d);
      if (d != 0.0f) allzero = false;
    }
    if (gH[r] == 0.0f) CHECK(allzero, "selective backward zero row %ld", long(r));
    else CHECK(std::fabs(s) <= rel * sa + 1e-6 && sa > 0.0, "selective backward row %ld sums to 0", long(r));
  }

  for (void* ptr : {dz_in, static_cast<void*>(d_ids), static_cast<void*>(d_old),
                    static_cast<void*>(d_adv), static_cast<void*>(d_mask), static_cast<void*>(d_w),
                    static_cast<void*>(d_loss), static_cast<void*>(d_logp),
                    static_cast<void*>(d_lse), static_cast<void*>(d_H), static_cast<void*>(d_clip),
                    static_cast<void*>(d_zero), d_dl, static_cast<void*>(d_lp2),
                    static_cast<void*>(d_lse2), static_cast<void*>(d_H2),
                    static_cast<void*>(d_gH)})
    HIP(hipFree(ptr));
  std::printf("case dtype=%s B=%ld L=%ld V=%ld T=%g done\n", dtype == GRPO_BF16 ? "bf16" : "f32",
              long(B), long(L), long(V), double(T));
}

// One fused-linear chunk called twice on the same inputs: the products and
// reductions are deterministic and loss_accum / grad_weight accumulate, so the
// second call doubles both exactly (x + x is exact in fp32); grad_hidden is
// overwritten (identical both times) and exactly zero on rows of weight 0.
static void run_fused() {
  const int64_t nseq = 2, L = 8, H = 64, V = 256, N = nseq * L;
  uint64_t seed = 777;
  std::vector<uint16_t> h(size_t(N * H)), W(size_t(V * H));
  for (auto& x : h) x = to_bf16(unif(seed, -1.0f, 1.0f));
  for (auto& x : W) x = to_bf16(unif(seed, -0.1f, 0.1f));
  std::vector<int64_t> ids(N);
  for (auto& y : ids) y = int64_t(lcg(seed) % uint32_t(V));
  std::vector<float> old(N), ref(N);
  for (auto& o : old) o = -std::log(float(V)) + unif(seed, -0.3f, 0.3f);
  for (auto& o : ref) o = -std::log(float(V)) + unif(seed, -0.1f, 0.1f);
  const std::vector<float> adv = {0.8f, 0.0f};
  std::vector<uint8_t> mask(N, 1);
  for (int64_t t = L - 3; t < L; ++t) mask[L + t] = 0;

  uint16_t* d_h = upload(h);
  uint16_t* d_W = upload(W);
  int64_t* d_ids = upload(ids);
  float *d_old = upload(old), *d_ref = upload(ref), *d_adv = upload(adv);
  uint8_t* d_mask = upload(mask);
  float* d_w = dalloc<float>(N);
  OK(grpo_loss_weights(d_mask, nseq, L, GRPO_REDUCE_TOKEN, d_w, nullptr));
  const size_t ws = fused_linear_grpo_workspace_bytes(N, V, H);
  CHECK(ws > 0, "workspace size");
  void* d_ws = dalloc<uint8_t>(ws);
  float* d_loss = dalloc<float>(1);
  float* d_gh = dalloc<float>(size_t(N * H));
  float* d_gW = dalloc<float>(size_t(V * H));
  HIP(hipMemset(d_loss, 0, sizeof(float)));
  HIP(hipMemset(d_gW, 0, size_t(V * H) * sizeof(float)));
  grpo_params p = {0.9f, 0.04f, 0.2f, 0.28f, GRPO_TOKEN, 0};

  OK(fused_linear_grpo_chunk(d_h, nseq, L, H, d_W, V, d_ids, d_old, d_ref, d_adv, d_mask, d_w,
                             &p, d_loss, d_gh, d_gW, d_ws, ws, nullptr));
  HIP(hipDeviceSynchronize());
  const auto loss1 = download(d_loss, 1), gh1 = download(d_gh, size_t(N * H)),
             gW1 = download(d_gW, size_t(V * H)), w = download(d_w, N);
  OK(fused_linear_grpo_chunk(d_h, nseq, L, H, d_W, V, d_ids, d_old, d_ref, d_adv, d_mask, d_w,
                             &p, d_loss, d_gh, d_gW, d_ws, ws, nullptr));
  HIP(hipDeviceSynchronize());
  const auto loss2 = download(d_loss, 1), gh2 = download(d_gh, size_t(N * H)),
             gW2 = download(d_gW, size_t(V * H));

  CHECK(std::isfinite(loss1[0]) && loss2[0] == 2.0f * loss1[0], "loss accumulates (%g, %g)",
        double(loss1[0]), double(loss2[0]));
  bool gW_ok = true, gW_nonzero = false;
  for (size_t i = 0; i < gW1.size(); ++i) {
    if (!std::isfinite(gW1[i]) || gW2[i] != 2.0f * gW1[i]) gW_ok = false;
    if (gW1[i] != 0.0f) gW_nonzero = true;
  }
  CHECK(gW_ok, "grad_weight accumulates exactly");
  CHECK(gW_nonzero, "grad_weight is not all zero");
  for (int64_t r = 0; r < N; ++r) {
    bool same = true, allzero = true;
    for (int64_t c = 0; c < H; ++c) {
      const float a = gh1[size_t(r * H + c)], b = gh2[size_t(r * H + c)];
      if (!(std::isfinite(a) && a == b)) same = false;
      if (a != 0.0f) allzero = false;
    }
    CHECK(same, "grad_hidden row %ld overwritten identically", long(r));
    if (w[r] == 0.0f) CHECK(allzero, "grad_hidden row %ld of weight 0 is zero", long(r));
  }
  for (void* ptr : {static_cast<void*>(d_h), static_cast<void*>(d_W), static_cast<void*>(d_ids),
                    static_cast<void*>(d_old), static_cast<void*>(d_ref),
                    static_cast<void*>(d_adv), static_cast<void*>(d_mask),
                    static_cast<void*>(d_w), d_ws, static_cast<void*>(d_loss),
                    static_cast<void*>(d_gh), static_cast<void*>(d_gW)})
    HIP(hipFree(ptr));
  std::printf("fused chunk nseq=%ld L=%ld H=%ld V=%ld done\n", long(nseq), long(L), long(H),
              long(V));
}

int main() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
    std::fprintf(stderr, "no GPU\n");
    return 2;
  }
  // argument errors come back before anything is enqueued
  CHECK(entropy_from_logits(nullptr, GRPO_BF16, 4, 100, 100, 1.0f, nullptr, nullptr) == GRPO_ERR_NULL,
        "NULL logits -> GRPO_ERR_NULL");
  CHECK(std::strlen(grpo_status_string(GRPO_ERR_SHAPE)) > 0, "status string");

  run_case(GRPO_F32, 3, 40, 1003, 0.9f);
  run_case(GRPO_BF16, 3, 40, 4096, 1.0f);
  run_fused();

  // group advantages of {1, 0, 0, 1}: +-(1/2) / (sqrt(1/3) + 1e-4)
  const std::vector<float> rw = {1, 0, 0, 1};
  float* d_r = upload(rw);
  float* d_a = dalloc<float>(4);
  OK(grpo_group_advantages(d_r, 4, 4, 1e-4f, 1, d_a, nullptr));
  const auto a = download(d_a, 4);
  const double want = 0.5 / (std::sqrt(1.0 / 3.0) + 1e-4);
  for (int i = 0; i < 4; ++i)
    CHECK(std::fabs(a[i] - (i == 0 || i == 3 ? want : -want)) <= 1e-6 * want, "advantage %d", i);
  HIP(hipFree(d_r));
  HIP(hipFree(d_a));

  if (failures) {
    std::fprintf(stderr, "abi_check: %d failures\n", failures);
    return 1;
  }
  std::printf("abi_check ok\n");
  return 0;
}
