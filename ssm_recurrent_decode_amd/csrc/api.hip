// Library-wide C ABI helpers (version, error strings, ring sizing) and the
// streaming HBM probes used to calibrate traffic counters.
#include "common.hpp"

namespace rssm {

struct CopyParams {
  float4* dst;
  const float4* src;
  size_t n16;
};

// Loads in flight per thread per pass of the probes (issued before any use).
constexpr int kProbeUnroll = 4;

// Grid-stride float4 copy: one read and one write of every byte, non-temporal
// like the decode kernels' state transfers (each wave instruction covers 1 KB).
__global__ __launch_bounds__(kBlock) void probe_copy_kernel(CopyParams p) {
  const size_t stride = (size_t)gridDim.x * kBlock * kProbeUnroll;
  for (size_t i = (size_t)blockIdx.x * kBlock * kProbeUnroll + threadIdx.x; i < p.n16; i += stride) {
    float4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      if (i + (size_t)u * kBlock < p.n16) v[u] = ld_f4_nt(reinterpret_cast<const float*>(p.src + i + (size_t)u * kBlock));
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      if (i + (size_t)u * kBlock < p.n16) st_f4_nt(reinterpret_cast<float*>(p.dst + i + (size_t)u * kBlock), v[u]);
  }
}

struct ReadParams {
  const float4* src;
  float* sink;
  size_t n16;
};

constexpr int kProbeBlocks = 4096;

// Grid-stride float4 read (non-temporal); one checksum per work-group keeps the
// loads live.
__global__ __launch_bounds__(kBlock) void probe_read_kernel(ReadParams p) {
  __shared__ float red[kBlock / kWave];
  const size_t stride = (size_t)gridDim.x * kBlock * kProbeUnroll;
  float acc = 0.f;
  for (size_t i = (size_t)blockIdx.x * kBlock * kProbeUnroll + threadIdx.x; i < p.n16; i += stride) {
    float4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      v[u] = (i + (size_t)u * kBlock < p.n16) ? ld_f4_nt(reinterpret_cast<const float*>(p.src + i + (size_t)u * kBlock))
                                              : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) p.sink[blockIdx.x] = red[0] + red[1] + red[2] + red[3];
}

}  // namespace rssm

extern "C" int rssm_abi_version(void) { return RSSM_ABI_VERSION; }

extern "C" const char* rssm_strerror(int code) {
  switch (code) {
    case RSSM_OK: return "ok";
    case RSSM_EINVAL: return "invalid argument (null pointer, bad or inconsistent size)";
    case RSSM_ENOTSUP:
      return "shape not compiled into this library (d in {64,128}; n in {64,128,256}; L <= 32, T <= 8)";
    case RSSM_ELAUNCH: return "HIP kernel launch failed";
    default: return "unknown error code";
  }
}

extern "C" int rssm_ring_sizes(const rssm_dims* d, int is_gdn, size_t out[4]) {
  if (!rssm_host::dims_ok(d) || d->capacity < 1 || out == nullptr) return RSSM_EINVAL;
  if (d->capacity > rssm::kMaxL) return RSSM_ENOTSUP;
  const size_t B = d->batch, H = d->nheads, G = d->ngroups, L = d->capacity;
  const size_t D = d->head_dim, N = d->state_dim;
  out[0] = B * H * L * D * ((is_gdn && !(d->flags & RSSM_F_U_BF16)) ? 4 : 2);
  out[1] = B * G * L * N * 2;
  out[2] = B * H * (size_t)rssm::meta_words((int)L) * 4;
  out[3] = 4;
  return RSSM_OK;
}

extern "C" int rssm_probe_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src || bytes == 0 || bytes % 16 != 0 || !rssm_host::aligned16(static_cast<const char*>(dst), static_cast<const char*>(src)))
    return RSSM_EINVAL;
  rssm::CopyParams p{static_cast<float4*>(dst), static_cast<const float4*>(src), bytes / 16};
  const size_t per_block = (size_t)rssm::kBlock * rssm::kProbeUnroll;
  const size_t want = (p.n16 + per_block - 1) / per_block;
  const dim3 grid((unsigned)(want < rssm::kProbeBlocks ? want : rssm::kProbeBlocks));
  return rssm_host::launch(rssm::probe_copy_kernel, grid, dim3(rssm::kBlock), stream, p);
}

extern "C" size_t rssm_probe_read_sink_floats(size_t bytes) {
  const size_t per_block = (size_t)rssm::kBlock * rssm::kProbeUnroll;
  const size_t want = (bytes / 16 + per_block - 1) / per_block;
  return want < (size_t)rssm::kProbeBlocks ? (want ? want : 1) : (size_t)rssm::kProbeBlocks;
}

extern "C" int rssm_probe_read(const void* src, size_t bytes, float* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || !rssm_host::aligned16(static_cast<const char*>(src), sink))
    return RSSM_EINVAL;
  rssm::ReadParams p{static_cast<const float4*>(src), sink, bytes / 16};
  const dim3 grid((unsigned)rssm_probe_read_sink_floats(bytes));
  return rssm_host::launch(rssm::probe_read_kernel, grid, dim3(rssm::kBlock), stream, p);
}
