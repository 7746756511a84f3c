// Fused causal depthwise conv1d state update with SiLU for gfx950.
//
// The conv state is channel-major with the time axis fastest (the "DS" layout of
// the vLLM disaggregated-serving page), bf16 [B, C, W-1].  With W = 4 a channel's
// state is 3 bf16 = 6 bytes, so one thread takes two consecutive channels: 12
// bytes of state (three aligned 4-byte words), 4 bytes of x, 16 bytes of taps,
// and writes 12 bytes of state and 8 bytes of fp32 output.  Consecutive threads
// touch consecutive bytes, so every access is coalesced.  The whole update is one
// memory round trip per thread; two channels per thread (B * C / 2 threads) beat
// four (3.87 vs 4.06 us at B = 256, C = 3072, graph-timed) and one (4.75 us).
#include "common.hpp"

namespace rssm {

struct ConvParams {
  uint16_t* state;
  const uint16_t* x;
  const uint16_t* w;
  float* out;
  int B, C;
};

__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }

__global__ __launch_bounds__(kBlock) void conv1d_update_w4_kernel(ConvParams p) {
  const int pairs = p.C >> 1;
  const long long t = (long long)blockIdx.x * kBlock + threadIdx.x;
  if (t >= (long long)p.B * pairs) return;
  const int b = (int)(t / pairs);
  const int c0 = (int)(t - (long long)b * pairs) * 2;

  uint32_t* st = reinterpret_cast<uint32_t*>(p.state + ((size_t)b * p.C + c0) * 3);
  const uint32_t s0 = st[0], s1 = st[1], s2 = st[2];
  const uint32_t xx = *reinterpret_cast<const uint32_t*>(p.x + (size_t)b * p.C + c0);
  const uint4 wq = *reinterpret_cast<const uint4*>(p.w + (size_t)c0 * 4);

  // channel m's window: state elements 3m .. 3m+2 (oldest first), then its x
  const uint32_t sv[6] = {s0 & 0xffffu, s0 >> 16, s1 & 0xffffu, s1 >> 16, s2 & 0xffffu, s2 >> 16};
  const uint32_t xv[2] = {xx & 0xffffu, xx >> 16};
  const uint32_t wv[8] = {wq.x & 0xffffu, wq.x >> 16, wq.y & 0xffffu, wq.y >> 16,
                          wq.z & 0xffffu, wq.z >> 16, wq.w & 0xffffu, wq.w >> 16};
  float o[2];
  uint32_t ns[6];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint32_t win[4] = {sv[3 * m], sv[3 * m + 1], sv[3 * m + 2], xv[m]};
    float z = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) z += bf16_to_f32(wv[4 * m + k]) * bf16_to_f32(win[k]);
    o[m] = silu(z);
    ns[3 * m] = win[1];
    ns[3 * m + 1] = win[2];
    ns[3 * m + 2] = win[3];
  }
  // written once and not read again by this launch: non-temporal stores, which keep
  // them from displacing the following kernel's lines in L2 (3.60 vs 3.76 us for the
  // update, 59.1 vs 59.7 us for the layer step with the append after it)
  float* op = p.out + (size_t)b * p.C + c0;
  __builtin_nontemporal_store(o[0], op);
  __builtin_nontemporal_store(o[1], op + 1);
  __builtin_nontemporal_store(ns[0] | (ns[1] << 16), st);
  __builtin_nontemporal_store(ns[2] | (ns[3] << 16), st + 1);
  __builtin_nontemporal_store(ns[4] | (ns[5] << 16), st + 2);
}

}  // namespace rssm

extern "C" int causal_conv1d_update(int32_t batch, int32_t channels, int32_t width,
                                    uint16_t* conv_state, const uint16_t* x, const uint16_t* weight,
                                    float* out, void* stream) {
  if (batch < 1 || channels < 1 || width < 2 || !conv_state || !x || !weight || !out ||
      !rssm_host::aligned16(conv_state, x, weight, out))
    return RSSM_EINVAL;
  if (width != 4 || channels % 2 != 0) return RSSM_ENOTSUP;
  rssm::ConvParams p{conv_state, x, weight, out, batch, channels};
  const long long threads = (long long)batch * (channels / 2);
  if (threads > (1LL << 31) - rssm::kBlock) return RSSM_EINVAL;
  const dim3 grid((unsigned)((threads + rssm::kBlock - 1) / rssm::kBlock));
  return rssm_host::launch(rssm::conv1d_update_w4_kernel, grid, dim3(rssm::kBlock), stream, p);
}
