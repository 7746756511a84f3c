// Gated DeltaNet decode kernels for gfx950: the standard step with state
// write-back, ReplaySSM chunk-wise speculative verify and the explicit flush.
//
// Method: "ReplaySSM: Cache SSM Inputs, Not State" -- background (the delta rule
// with its Householder term) and appendix (GDN standard decode: cache the
// correction u so the update becomes S_t = alpha_t S_{t-1} + u_t k_t^T; GDN
// speculative decoding: all T corrections of a window from one strictly
// lower-triangular T x T solve).
//
// Work decomposition: one work-group of four waves per (request, head), the state
// in the tile layout of common.hpp.  The verify kernel itself is in gdn.hpp.
#include "gdn.hpp"

namespace rssm {

// ======================================================= standard GDN step
struct GdnStdParams {
  float* state;
  const uint16_t* v;
  const uint16_t* k;
  const uint16_t* q;
  const float* g;
  const float* beta;
  float* y;
  int H, G;
};

// u = beta (v - alpha S k);  S <- alpha S + u k^T;  y = S q;  S written back.
template <int D, int N>
__global__ __launch_bounds__(kBlock) void gdn_step_kernel(GdnStdParams p) {
  constexpr int NCT = N / 16;
  constexpr int RT = D / (16 * kWavesPerBlock);
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int b = wg / p.H, h = wg - b * p.H, g = h / (p.H / p.G);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, cq = lane >> 4;

  float* S = p.state + (size_t)wg * D * N;
  float4 s[RT][NCT];  // line arrangement until each pair is settled
  load_state_lines<N, RT, NCT>(s, S, wave, r, cq);
  const uint16_t* kp = p.k + ((size_t)b * p.G + g) * N + cq * 4;
  const uint16_t* qp = p.q + ((size_t)b * p.G + g) * N + cq * 4;
  uint2 kk[NCT], qq[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    kk[ct] = ld_u2(kp + ct * 16);
    qq[ct] = ld_u2(qp + ct * 16);
  }
  float vr[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) vr[rt] = bf16_to_f32(p.v[(size_t)wg * D + (wave * RT + rt) * 16 + r]);
  const float alpha = expf(p.g[wg]);
  const float beta = p.beta[wg];

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
    float sk = 0.f;
#pragma unroll
    for (int jj = 0; jj < NCT / 2; ++jj) {
      settle_pair(s[rt][2 * jj], s[rt][2 * jj + 1]);
      sk += dot4_bf16(s[rt][2 * jj], kk[2 * jj]) + dot4_bf16(s[rt][2 * jj + 1], kk[2 * jj + 1]);
    }
    sk = reduce_row4(sk);
    const float u = beta * (vr[rt] - alpha * sk);
    float acc = 0.f;
#pragma unroll
    for (int jj = 0; jj < NCT / 2; ++jj) {
      float4 xo[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ct = 2 * jj + half;
        float4 x = s[rt][ct];
        x.x = alpha * x.x + u * bf16_lo(kk[ct].x);
        x.y = alpha * x.y + u * bf16_hi(kk[ct].x);
        x.z = alpha * x.z + u * bf16_lo(kk[ct].y);
        x.w = alpha * x.w + u * bf16_hi(kk[ct].y);
        acc += dot4_bf16(x, qq[ct]);
        xo[half] = x;
      }
      store_pair_lines<N>(S, wave * RT + rt, jj, xo[0], xo[1], r, cq);
    }
    acc = reduce_row4(acc);
    if (cq == 0) p.y[(size_t)wg * D + row] = acc;
  }
}

// ======================================================= ReplaySSM GDN
// Explicit GDN flush of the committed entries of masked requests.
template <int D, int N, bool EAGER>
__global__ __launch_bounds__(kBlock) void gdn_flush_kernel(GdnReplayParams p) {
  constexpr int NCT = N / 16;
  constexpr int RT = D / (16 * kWavesPerBlock);
  __shared__ float s_w[kMaxL];
  __shared__ float s_abar;
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kMaxL * N];
  __shared__ __attribute__((aligned(16))) float s_u[kMaxL * D];

  const int H = p.H, G = p.G, L = p.L;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int b = wg / H, h = wg - b * H, g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, cq = lane >> 4;

  if (p.mask != nullptr && p.mask[b] == 0) return;
  const int rb = pool_row(p.slots, p.rows, b, p.err, tid == 0 && h == 0);
  if (rb < 0) return;
  const size_t bh = (size_t)rb * H + h;
  float* rec = p.meta + bh * meta_words(L);  // this head's ring record
  // read per lane, so that the eager checkpoint loads below are issued before it arrives
  const unsigned long long word = *reinterpret_cast<const unsigned long long*>(rec + kMetaPtr + opaque_zero());
  // EAGER (no mask: every request that holds entries folds them): the checkpoint
  // is requested before the pointer word is known, one memory round trip earlier
  // (a request whose ring is empty reads it in vain).  With a mask it is requested
  // only for requests that fold.
  float* S0 = p.state0 + bh * D * N;
  float4 s[RT][NCT];
  if constexpr (EAGER) load_state_lines<N, RT, NCT>(s, S0, wave, r, cq);
  const RingPtr rp = unpack_ptr(word);
  int head = rp.head, cnt = rp.count;
  int bad = 0;
  if (head >= L) {
    head %= L;
    bad |= RSSM_ERR_POINTERS;
  }
  if (cnt > L) {
    cnt = L;
    bad |= RSSM_ERR_POINTERS;
  }
  if (cnt + rp.pending > L) bad |= RSSM_ERR_POINTERS;
  const int F = cnt;
  if (!EAGER && F > 0) load_state_lines<N, RT, NCT>(s, S0, wave, r, cq);
  // the F entries' corrections and keys into LDS by logical index, 16 bytes per
  // thread, every load issued before the first one is waited for (one round trip)
  constexpr int KCH = N / 8;  // 16-byte chunks of a key
  constexpr int UP = (kMaxL * (D / 4) + kBlock - 1) / kBlock, KP = (kMaxL * KCH + kBlock - 1) / kBlock;
  const int cpe = p.u_bf16 ? D / 8 : D / 4;  // 16-byte chunks of a cached correction
  uint4 uc[UP], kc[KP];
#pragma unroll
  for (int i = 0; i < UP; ++i) {
    const int t = tid + i * kBlock, j = t / cpe;
    if (j < F) {
      const size_t e = ring_entry(rb, h, H, L, (head + j) % L, D);
      uc[i] = p.u_bf16 ? ld_u4(reinterpret_cast<const uint16_t*>(p.ring_u) + e + (t % cpe) * 8)
                       : *reinterpret_cast<const uint4*>(p.ring_u + e + (t % cpe) * 4);
    }
  }
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int t = tid + i * kBlock, j = t / KCH;
    if (j < F) kc[i] = ld_u4(p.ring_k + (((size_t)rb * G + g) * L + (head + j) % L) * N + (t % KCH) * 8);
  }
  if (wave == 0) {
    const int j = lane;
    const float al_rec = rec[kMetaSlot + (head + min(j, L - 1)) % L];  // read unconditionally
    const float al = (j < F) ? al_rec : 1.f;
    float R = 1.f, P = 1.f;
    for (int m = 0; m < F; ++m) {
      const float am = __shfl(al, m, kWave);
      P *= am;
      if (m > j) R *= am;
    }
    if (j < F) s_w[j] = R;
    if (lane == 0) s_abar = P;
  }
#pragma unroll
  for (int i = 0; i < UP; ++i) {
    const int t = tid + i * kBlock, j = t / cpe;
    if (j < F) {
      float* dst = &s_u[j * D];
      if (p.u_bf16) {
        const int o = (t % cpe) * 8;
        *reinterpret_cast<float4*>(dst + o) =
            make_float4(bf16_lo(uc[i].x), bf16_hi(uc[i].x), bf16_lo(uc[i].y), bf16_hi(uc[i].y));
        *reinterpret_cast<float4*>(dst + o + 4) =
            make_float4(bf16_lo(uc[i].z), bf16_hi(uc[i].z), bf16_lo(uc[i].w), bf16_hi(uc[i].w));
      } else {
        *reinterpret_cast<uint4*>(dst + (t % cpe) * 4) = uc[i];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int t = tid + i * kBlock, j = t / KCH;
    if (j < F) *reinterpret_cast<uint4*>(&s_k[j * N + (t % KCH) * 8]) = kc[i];
  }
  __syncthreads();
  float uf[RT][kVJ];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
    for (int m = 0; m < kVJ; ++m) {
      const int j = cq + 4 * m;
      uf[rt][m] = (j < F) ? s_u[j * D + row] : 0.f;
    }
  }
  if (F > 0) {
    settle_state<RT, NCT>(s);
    fold_and_store<D, N, RT, NCT, kVJ>(S0, s, s_abar, s_k, s_w, uf, F, wave, r, cq);
  }

  if (tid == 0) {
    if (h == 0) flag_error(p.err, bad);
    *reinterpret_cast<unsigned long long*>(rec + kMetaPtr) = pack_ptr((head + F) % L, 0, rp.pending);
  }
}

}  // namespace rssm

using namespace rssm;
using rssm_host::launch;

namespace {

GdnReplayParams make_gdn_params(const rssm_dims* d, float* state0, rssm_ring* ring) {
  GdnReplayParams p{};
  p.state0 = state0;
  p.ring_u = static_cast<float*>(ring->vu);
  p.ring_k = ring->k;
  p.meta = reinterpret_cast<float*>(ring->meta);
  p.err = ring->err;
  p.slots = ring->slots;
  p.rows = ring->rows;
  p.y_bf16 = (d->flags & RSSM_F_Y_BF16) != 0;
  p.u_bf16 = (d->flags & RSSM_F_U_BF16) != 0;
  p.H = d->nheads;
  p.G = d->ngroups;
  p.L = d->capacity;
  return p;
}

}  // namespace

extern "C" int gdn_decode_step(const rssm_dims* dims, float* state, const uint16_t* v,
                               const uint16_t* k, const uint16_t* q, const float* g,
                               const float* beta, float* y, void* stream) {
  if (!rssm_host::dims_ok(dims) || !state || !v || !k || !q || !g || !beta || !y ||
      !rssm_host::aligned16(state, v, k, q, g, beta, y))
    return RSSM_EINVAL;
  if (!rssm_host::shape_supported(dims) || (dims->flags & RSSM_F_Y_BF16)) return RSSM_ENOTSUP;
  GdnStdParams p{state, v, k, q, g, beta, y, dims->nheads, dims->ngroups};
  const dim3 grid(dims->batch * dims->nheads);
  const bool d64 = dims->head_dim == 64;
  switch (dims->state_dim) {
    case 64: return launch(d64 ? gdn_step_kernel<64, 64> : gdn_step_kernel<128, 64>, grid, dim3(kBlock), stream, p);
    case 256: return launch(d64 ? gdn_step_kernel<64, 256> : gdn_step_kernel<128, 256>, grid, dim3(kBlock), stream, p);
    default: return launch(d64 ? gdn_step_kernel<64, 128> : gdn_step_kernel<128, 128>, grid, dim3(kBlock), stream, p);
  }
}

namespace {

int gdn_verify_common(const rssm_dims* dims, int32_t T, float* state0, rssm_ring* ring, const int32_t* accepted,
                      const uint16_t* v, const uint16_t* k, const uint16_t* q, const float* g,
                      const float* beta, float* y, int32_t* flushed, void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::ring_ok(ring) || !state0 || !v || !k || !q ||
      !g || !beta || !y || !rssm_host::aligned16(state0, v, k, q, g, beta, y, flushed))
    return RSSM_EINVAL;
  if (T < 1 || dims->capacity < 2 * T) return RSSM_EINVAL;
  if (!rssm_host::ring_shape_supported(dims) || T > kMaxT) return RSSM_ENOTSUP;
  GdnReplayParams p = make_gdn_params(dims, state0, ring);
  p.accepted = accepted;
  p.v = v;
  p.k = k;
  p.q = q;
  p.g = g;
  p.beta = beta;
  p.y = y;
  p.flushed = flushed;
  const int D = dims->head_dim;
  if (dims->state_dim == 64) return rssm_host::launch_gdn_n64(T, D, p, dims->batch, stream);
  if (dims->state_dim == 256) return rssm_host::launch_gdn_n256(T, D, p, dims->batch, stream);
  if (T <= 4) return rssm_host::launch_gdn_verify_lo(T, D, p, dims->batch, stream);
  return rssm_host::launch_gdn_verify_hi(T, D, p, dims->batch, stream);
}

}  // namespace

extern "C" int gdn_replay_verify_T(const rssm_dims* dims, int32_t T, float* state0, rssm_ring* ring,
                                   const uint16_t* v, const uint16_t* k, const uint16_t* q,
                                   const float* g, const float* beta, float* y, int32_t* flushed,
                                   void* stream) {
  return gdn_verify_common(dims, T, state0, ring, nullptr, v, k, q, g, beta, y, flushed, stream);
}

extern "C" int gdn_replay_commit_verify_T(const rssm_dims* dims, int32_t T, float* state0, rssm_ring* ring,
                                          const int32_t* accepted, const uint16_t* v, const uint16_t* k,
                                          const uint16_t* q, const float* g, const float* beta, float* y,
                                          int32_t* flushed, void* stream) {
  if (!accepted || !rssm_host::aligned16(accepted)) return RSSM_EINVAL;
  return gdn_verify_common(dims, T, state0, ring, accepted, v, k, q, g, beta, y, flushed, stream);
}

extern "C" int gdn_replay_append_decode(const rssm_dims* dims, float* state0, rssm_ring* ring,
                                        const uint16_t* v, const uint16_t* k, const uint16_t* q,
                                        const float* g, const float* beta, float* y, int32_t* flushed,
                                        void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::ring_ok(ring) || !state0 || !v || !k || !q ||
      !g || !beta || !y || !rssm_host::aligned16(state0, v, k, q, g, beta, y, flushed))
    return RSSM_EINVAL;
  if (dims->capacity < 1) return RSSM_EINVAL;
  if (!rssm_host::ring_shape_supported(dims)) return RSSM_ENOTSUP;
  GdnReplayParams p = make_gdn_params(dims, state0, ring);
  p.v = v;
  p.k = k;
  p.q = q;
  p.g = g;
  p.beta = beta;
  p.y = y;
  p.flushed = flushed;
  if (dims->state_dim == 64) return rssm_host::launch_gdn_n64(0, dims->head_dim, p, dims->batch, stream);
  if (dims->state_dim == 256) return rssm_host::launch_gdn_n256(0, dims->head_dim, p, dims->batch, stream);
  if (dims->head_dim == 64) return rssm_host::launch_gdn_window<64, 1, true>(p, dims->batch, stream);
  return rssm_host::launch_gdn_window<128, 1, true>(p, dims->batch, stream);
}

namespace {

// the flush instances of one mode: EAGER when no mask selects the requests
template <bool EAGER>
int launch_gdn_replay_flush(const rssm_dims* dims, const GdnReplayParams& p, void* stream) {
  const dim3 grid(dims->batch * dims->nheads);
  const bool d64 = dims->head_dim == 64;
  switch (dims->state_dim) {
    case 64:
      return launch(d64 ? gdn_flush_kernel<64, 64, EAGER> : gdn_flush_kernel<128, 64, EAGER>, grid, dim3(kBlock),
                    stream, p);
    case 256:
      return launch(d64 ? gdn_flush_kernel<64, 256, EAGER> : gdn_flush_kernel<128, 256, EAGER>, grid, dim3(kBlock),
                    stream, p);
    default:
      return launch(d64 ? gdn_flush_kernel<64, 128, EAGER> : gdn_flush_kernel<128, 128, EAGER>, grid, dim3(kBlock),
                    stream, p);
  }
}

}  // namespace

extern "C" int gdn_replay_flush(const rssm_dims* dims, float* state0, rssm_ring* ring,
                                const int32_t* mask, void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::ring_ok(ring) || !state0 ||
      !rssm_host::aligned16(state0, mask))
    return RSSM_EINVAL;
  if (dims->capacity < 1) return RSSM_EINVAL;
  if (!rssm_host::ring_shape_supported(dims)) return RSSM_ENOTSUP;
  GdnReplayParams p = make_gdn_params(dims, state0, ring);
  p.mask = mask;
  return mask == nullptr ? launch_gdn_replay_flush<true>(dims, p, stream)
                         : launch_gdn_replay_flush<false>(dims, p, stream);
}
