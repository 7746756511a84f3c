// Fused causal depthwise conv1d state update with SiLU for gfx950.
//
// The conv state is channel-major with the time axis fastest (the "DS" layout of
// the vLLM disaggregated-serving page), bf16 [B, C, W-1].  With W = 4 a channel's
// state is 3 bf16 = 6 bytes, so one thread takes four consecutive channels: 24
// bytes of state (three aligned 8-byte loads), 8 bytes of x, 32 bytes of taps, and
// writes 24 bytes of state and 16 bytes of fp32 output.  Consecutive threads touch
// consecutive bytes, so every access is coalesced.
#include "common.hpp"

namespace rssm {

struct ConvParams {
  uint16_t* state;
  const uint16_t* x;
  const uint16_t* w;
  float* out;
  int B, C;
};

__device__ __forceinline__ uint32_t bf16_bits(uint2 v, int i) {
  const uint32_t word = (i < 2) ? v.x : v.y;
  return (i & 1) ? (word >> 16) : (word & 0xffffu);
}

__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }

__global__ __launch_bounds__(kBlock) void conv1d_update_w4_kernel(ConvParams p) {
  const int groups = p.C >> 2;
  const long long t = (long long)blockIdx.x * kBlock + threadIdx.x;
  if (t >= (long long)p.B * groups) return;
  const int b = (int)(t / groups);
  const int c0 = (int)(t - (long long)b * groups) * 4;

  uint16_t* st = p.state + ((size_t)b * p.C + c0) * 3;
  const uint2 s0 = *reinterpret_cast<const uint2*>(st);
  const uint2 s1 = *reinterpret_cast<const uint2*>(st + 4);
  const uint2 s2 = *reinterpret_cast<const uint2*>(st + 8);
  const uint2 xx = *reinterpret_cast<const uint2*>(p.x + (size_t)b * p.C + c0);
  const uint4 w0 = *reinterpret_cast<const uint4*>(p.w + (size_t)c0 * 4);
  const uint4 w1 = *reinterpret_cast<const uint4*>(p.w + (size_t)c0 * 4 + 8);

  // 12 state values: channel m owns elements 3m .. 3m+2 (oldest first)
  uint32_t sv[12];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sv[i] = bf16_bits(s0, i);
    sv[4 + i] = bf16_bits(s1, i);
    sv[8 + i] = bf16_bits(s2, i);
  }
  const uint32_t wv[16] = {w0.x & 0xffffu, w0.x >> 16, w0.y & 0xffffu, w0.y >> 16,
                           w0.z & 0xffffu, w0.z >> 16, w0.w & 0xffffu, w0.w >> 16,
                           w1.x & 0xffffu, w1.x >> 16, w1.y & 0xffffu, w1.y >> 16,
                           w1.z & 0xffffu, w1.z >> 16, w1.w & 0xffffu, w1.w >> 16};
  float o[4];
  uint32_t ns[12];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t xm = bf16_bits(xx, m);
    const uint32_t win[4] = {sv[3 * m], sv[3 * m + 1], sv[3 * m + 2], xm};
    float z = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) z += bf16_to_f32(wv[4 * m + k]) * bf16_to_f32(win[k]);
    o[m] = silu(z);
    ns[3 * m] = win[1];
    ns[3 * m + 1] = win[2];
    ns[3 * m + 2] = win[3];
  }
  *reinterpret_cast<float4*>(p.out + (size_t)b * p.C + c0) = make_float4(o[0], o[1], o[2], o[3]);
  *reinterpret_cast<uint2*>(st) = make_uint2(ns[0] | (ns[1] << 16), ns[2] | (ns[3] << 16));
  *reinterpret_cast<uint2*>(st + 4) = make_uint2(ns[4] | (ns[5] << 16), ns[6] | (ns[7] << 16));
  *reinterpret_cast<uint2*>(st + 8) = make_uint2(ns[8] | (ns[9] << 16), ns[10] | (ns[11] << 16));
}

}  // namespace rssm

extern "C" int causal_conv1d_update(int32_t batch, int32_t channels, int32_t width,
                                    uint16_t* conv_state, const uint16_t* x, const uint16_t* weight,
                                    float* out, void* stream) {
  if (batch < 1 || channels < 1 || width < 2 || !conv_state || !x || !weight || !out)
    return RSSM_EINVAL;
  if (width != 4 || channels % 4 != 0) return RSSM_ENOTSUP;
  rssm::ConvParams p{conv_state, x, weight, out, batch, channels};
  const long long threads = (long long)batch * (channels / 4);
  if (threads > (1LL << 31) - rssm::kBlock) return RSSM_EINVAL;
  const dim3 grid((unsigned)((threads + rssm::kBlock - 1) / rssm::kBlock));
  return rssm_host::launch(rssm::conv1d_update_w4_kernel, grid, dim3(rssm::kBlock), stream, p);
}
