// The C ABI used from C++ without Python or torch: buffers from hipMalloc, one HIP
// stream, the standard Mamba-2 step and ReplaySSM append-decode run side by side on
// the same inputs for 2L + 3 steps (two flushes).  ReplaySSM computes the same
// outputs as the recurrence it replaces, so the two y must agree (relative 1e-3 of
// the largest output), and the ring pointers must follow the flush-when-full
// schedule (count = (t + 1) mod L after step t, head advancing by L at a flush,
// i.e. staying 0): read per request through rssm_ring_pointers into device int32
// arrays, and cross-checked against the typed record of the last head of every
// request.  Exit status 0 and "ok" on success.  Built next to the library by
// ssm_recurrent_decode_amd.build.
//
// With a directory as the only argument, the program also writes what it fed the
// library and what came back, as raw little-endian arrays, for a comparison with
// the float64 oracle: S0.f32 [B,H,d,n], A.f32 [H], dt_bias.f32 [H], and per step,
// appended in step order, v.bf16 [B,H,d], k.bf16 / q.bf16 [B,G,n], dt.f32 [B,H],
// y_replay.f32 and y_standard.f32 [B,H,d].
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "ssm_recurrent_decode.h"

namespace {

#define CHECK_HIP(x)                                                         \
  do {                                                                       \
    hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                  \
      std::printf("HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      return 1;                                                              \
    }                                                                        \
  } while (0)

#define CHECK_RC(x)                                                          \
  do {                                                                       \
    int r_ = (x);                                                            \
    if (r_ != RSSM_OK) {                                                     \
      std::printf("%s failed: %s\n", #x, rssm_strerror(r_));                 \
      return 1;                                                              \
    }                                                                        \
  } while (0)

uint16_t bf16(float f) {  // round to nearest even
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

struct Lcg {  // uniform on [lo, hi), 64-bit linear congruential generator
  uint64_t s;
  float operator()(float lo, float hi) {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return lo + (hi - lo) * static_cast<float>((s >> 40) * (1.0 / 16777216.0));
  }
};

// Appends n elements of T to dir/name (no-op when dir is empty); false on error.
template <typename T>
bool dump(const std::string& dir, const char* name, const T* data, size_t n, bool first) {
  if (dir.empty()) return true;
  FILE* f = std::fopen((dir + "/" + name).c_str(), first ? "wb" : "ab");
  if (f == nullptr) return false;
  const bool ok = std::fwrite(data, sizeof(T), n, f) == n;
  return std::fclose(f) == 0 && ok;
}

}  // namespace

int main(int argc, char** argv) {
  const std::string out_dir = argc > 1 ? argv[1] : "";
#define CHECK_DUMP(x)                              \
  do {                                             \
    if (!(x)) {                                    \
      std::printf("cannot write %s\n", #x);        \
      return 1;                                    \
    }                                              \
  } while (0)
  const int B = 4, H = 8, D = 64, N = 128, G = 2, L = 8, steps = 2 * L + 3;
  rssm_dims dims{B, H, D, N, G, L, 0};
  if (rssm_abi_version() != RSSM_ABI_VERSION) {
    std::printf("ABI version mismatch\n");
    return 1;
  }
  size_t rs[4];
  CHECK_RC(rssm_ring_sizes(&dims, 0, rs));

  const size_t ns = (size_t)B * H * D * N;
  Lcg rng{20260601};
  std::vector<float> S(ns);
  for (auto& x : S) x = rng(-0.3f, 0.3f);
  std::vector<float> A(H), bias(H);
  for (int h = 0; h < H; ++h) {
    A[h] = -rng(0.5f, 8.f);
    bias[h] = rng(-4.f, -2.f);
  }

  float *state, *state0, *dA, *dbias, *ddt, *ys, *yr;
  uint16_t *dv, *dk, *dq;
  int32_t* dptr;  // [3][B]: head, count, pending
  void* ring_mem[4];
  CHECK_HIP(hipMalloc(&state, ns * 4));
  CHECK_HIP(hipMalloc(&state0, ns * 4));
  CHECK_HIP(hipMalloc(&dA, H * 4));
  CHECK_HIP(hipMalloc(&dbias, H * 4));
  CHECK_HIP(hipMalloc(&ddt, B * H * 4));
  CHECK_HIP(hipMalloc(&ys, (size_t)B * H * D * 4));
  CHECK_HIP(hipMalloc(&yr, (size_t)B * H * D * 4));
  CHECK_HIP(hipMalloc(&dv, (size_t)B * H * D * 2));
  CHECK_HIP(hipMalloc(&dk, (size_t)B * G * N * 2));
  CHECK_HIP(hipMalloc(&dq, (size_t)B * G * N * 2));
  CHECK_HIP(hipMalloc(&dptr, 3 * B * 4));
  for (int i = 0; i < 4; ++i) {
    CHECK_HIP(hipMalloc(&ring_mem[i], rs[i]));
    CHECK_HIP(hipMemset(ring_mem[i], 0, rs[i]));
  }
  CHECK_HIP(hipMemcpy(state, S.data(), ns * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(state0, S.data(), ns * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dA, A.data(), H * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dbias, bias.data(), H * 4, hipMemcpyHostToDevice));
  CHECK_DUMP(dump(out_dir, "S0.f32", S.data(), S.size(), true));
  CHECK_DUMP(dump(out_dir, "A.f32", A.data(), A.size(), true));
  CHECK_DUMP(dump(out_dir, "dt_bias.f32", bias.data(), bias.size(), true));
  rssm_ring ring{ring_mem[0], static_cast<uint16_t*>(ring_mem[1]), static_cast<rssm_ring_record*>(ring_mem[2]),
                 static_cast<int32_t*>(ring_mem[3]), nullptr, 0};
  const size_t lines = RSSM_RECORD_LINES(L);  // 128-byte lines per (request, head) record
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  std::vector<uint16_t> v((size_t)B * H * D), k((size_t)B * G * N), q((size_t)B * G * N);
  std::vector<float> dt(B * H), hs((size_t)B * H * D), hr((size_t)B * H * D);
  const float ks = 1.f / std::sqrt((float)N);
  for (int t = 0; t < steps; ++t) {
    for (auto& x : v) x = bf16(rng(-1.f, 1.f));
    for (auto& x : k) x = bf16(rng(-ks, ks));
    for (auto& x : q) x = bf16(rng(-ks, ks));
    for (auto& x : dt) x = rng(-1.f, 1.f);
    CHECK_HIP(hipMemcpyAsync(dv, v.data(), v.size() * 2, hipMemcpyHostToDevice, stream));
    CHECK_HIP(hipMemcpyAsync(dk, k.data(), k.size() * 2, hipMemcpyHostToDevice, stream));
    CHECK_HIP(hipMemcpyAsync(dq, q.data(), q.size() * 2, hipMemcpyHostToDevice, stream));
    CHECK_HIP(hipMemcpyAsync(ddt, dt.data(), dt.size() * 4, hipMemcpyHostToDevice, stream));
    CHECK_RC(ssm_decode_step(&dims, state, dv, dk, dq, ddt, dbias, dA, ys, stream));
    CHECK_RC(replay_append_decode(&dims, state0, &ring, dv, dk, dq, ddt, dbias, dA, yr, nullptr, stream));
    CHECK_HIP(hipMemcpyAsync(hs.data(), ys, hs.size() * 4, hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipMemcpyAsync(hr.data(), yr, hr.size() * 4, hipMemcpyDeviceToHost, stream));
    CHECK_RC(rssm_ring_pointers(&dims, &ring, dptr, dptr + B, dptr + 2 * B, stream));
    int32_t ptrs[3 * B];
    CHECK_HIP(hipMemcpyAsync(ptrs, dptr, sizeof(ptrs), hipMemcpyDeviceToHost, stream));
    std::vector<rssm_ring_record> last(B);  // record of head H - 1 of every request
    for (int b = 0; b < B; ++b)
      CHECK_HIP(hipMemcpyAsync(&last[b], ring.meta + ((size_t)b * H + H - 1) * lines, sizeof(rssm_ring_record),
                               hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    CHECK_DUMP(dump(out_dir, "v.bf16", v.data(), v.size(), t == 0));
    CHECK_DUMP(dump(out_dir, "k.bf16", k.data(), k.size(), t == 0));
    CHECK_DUMP(dump(out_dir, "q.bf16", q.data(), q.size(), t == 0));
    CHECK_DUMP(dump(out_dir, "dt.f32", dt.data(), dt.size(), t == 0));
    CHECK_DUMP(dump(out_dir, "y_replay.f32", hr.data(), hr.size(), t == 0));
    CHECK_DUMP(dump(out_dir, "y_standard.f32", hs.data(), hs.size(), t == 0));
    double mx = 0.0, err = 0.0;
    for (size_t i = 0; i < hs.size(); ++i) {
      mx = std::fmax(mx, std::fabs((double)hs[i]));
      err = std::fmax(err, std::fabs((double)hs[i] - (double)hr[i]));
    }
    if (!(err <= 1e-3 * mx)) {
      std::printf("step %d: replay and standard outputs differ (max %g, largest |y| %g)\n", t, err, mx);
      return 1;
    }
    for (int b = 0; b < B; ++b) {
      const uint64_t w = last[b].ptr;
      if (ptrs[b] != 0 || ptrs[B + b] != (t + 1) % L || ptrs[2 * B + b] != 0 || RSSM_PTR_HEAD(w) != 0u ||
          RSSM_PTR_COUNT(w) != (uint32_t)ptrs[B + b] || RSSM_PTR_PENDING(w) != 0u) {
        std::printf("step %d request %d: pointers head %d count %d pending %d, last head's record %u/%u/%u\n", t, b,
                    ptrs[b], ptrs[B + b], ptrs[2 * B + b], RSSM_PTR_HEAD(w), RSSM_PTR_COUNT(w), RSSM_PTR_PENDING(w));
        return 1;
      }
    }
  }
  int32_t err_bits = -1;
  CHECK_HIP(hipMemcpy(&err_bits, ring.err, 4, hipMemcpyDeviceToHost));
  if (err_bits != 0) {
    std::printf("ring anomaly bits %d\n", err_bits);
    return 1;
  }
  CHECK_HIP(hipStreamDestroy(stream));
  std::printf("ok: %d steps, replay matches the standard step\n", steps);
  return 0;
}
