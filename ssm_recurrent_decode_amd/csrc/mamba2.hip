// Mamba-2 decode kernels for gfx950: the standard step with state write-back, and
// ReplaySSM append-decode / speculative verify / flush / rollback.
//
// Method: "ReplaySSM: Cache SSM Inputs, Not State" -- background (the recurrence),
// method (core idea, output-only decode, rollback as a pointer move), algorithms
// (Mamba-2 standard decode; speculative decoding with the early-flush rule) and
// kernel design (shared inner products, ring indexed in-kernel).
//
// Work decomposition: one work-group of four waves per (request b, head h).  Each
// wave streams D/64 row tiles of the head's d x n fp32 state, moved in the line
// arrangement and computed on in the tile layout described in common.hpp (one
// float4 per lane per 16x16 tile, all loads issued before any dependent
// arithmetic).  Work-groups are renumbered so that the heads
// of a request land on one XCD.
#include "replay.hpp"

namespace rssm {

// ======================================================= standard Mamba-2 step
struct StdParams {
  float* state;
  const uint16_t* v;
  const uint16_t* k;
  const uint16_t* q;
  const float* dt;
  const float* dt_bias;
  const float* A;
  float* y;
  int H, G;
};

// S <- a S + Delta v k^T ; y = S q ; S written back (the baseline that ReplaySSM
// improves on: 8dn bytes of state traffic per head).
template <int D, int N>
__global__ __launch_bounds__(kBlock) void ssm_step_kernel(StdParams p) {
  constexpr int NCT = N / 16;
  constexpr int RT = D / (16 * kWavesPerBlock);
  const int wg = xcd_remap(blockIdx.x, gridDim.x);  // == b * H + h
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
  const float delta = softplus_f32(p.dt[wg] + p.dt_bias[h]);
  const float a = expf(p.A[h] * delta);

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
    const float dv = delta * vr[rt];
    float acc = 0.f;
#pragma unroll
    for (int jj = 0; jj < NCT / 2; ++jj) {
      settle_pair(s[rt][2 * jj], s[rt][2 * jj + 1]);
      float4 xo[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int ct = 2 * jj + half;
        float4 x = s[rt][ct];
        x.x = a * x.x + dv * bf16_lo(kk[ct].x);
        x.y = a * x.y + dv * bf16_hi(kk[ct].x);
        x.z = a * x.z + dv * bf16_lo(kk[ct].y);
        x.w = a * x.w + dv * bf16_hi(kk[ct].y);
        acc += dot4_bf16(x, qq[ct]);
        xo[half] = x;
      }
      store_pair_lines<N>(S, wave * RT + rt, jj, xo[0], xo[1], r, cq);
    }
    acc = reduce_row4(acc);
    if (cq == 0) p.y[(size_t)wg * D + row] = acc;
  }
}

// Explicit flush of the committed entries of masked requests.
template <int D, int N, bool EAGER>
__global__ __launch_bounds__(kBlock) void replay_flush_kernel(ReplayParams p) {
  constexpr int NCT = N / 16;
  constexpr int RT = D / (16 * kWavesPerBlock);
  __shared__ float s_fw[kMaxL];
  __shared__ float s_fabar;
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kMaxL * N];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[kMaxL * D];

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
  // the F entries' values and keys into LDS by logical index, 16 bytes per thread,
  // every load issued before the first one is waited for (one round trip)
  constexpr int VCH = D / 8, KCH = N / 8;  // 16-byte chunks of a value, of a key
  constexpr int VP = (kMaxL * VCH + kBlock - 1) / kBlock, KP = (kMaxL * KCH + kBlock - 1) / kBlock;
  uint4 vc[VP], kc[KP];
#pragma unroll
  for (int i = 0; i < VP; ++i) {
    const int t = tid + i * kBlock, j = t / VCH;
    if (j < F) vc[i] = ld_u4(p.ring_v + ring_entry(rb, h, H, L, (head + j) % L, D) + (t % VCH) * 8);
  }
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int t = tid + i * kBlock, j = t / KCH;
    if (j < F) kc[i] = ld_u4(p.ring_k + (((size_t)rb * G + g) * L + (head + j) % L) * N + (t % KCH) * 8);
  }
  if (wave == 0) {
    const int j = lane;
    const float dl_rec = rec[kMetaSlot + (head + min(j, L - 1)) % L];  // read unconditionally
    const float dl = (j < F) ? dl_rec : 0.f;
    const float al = (j < F) ? expf(rec[kMetaA] * dl) : 1.f;
    float R = 1.f, P = 1.f;
    for (int m = 0; m < F; ++m) {
      const float am = __shfl(al, m, kWave);
      P *= am;
      if (m > j) R *= am;
    }
    if (j < F) s_fw[j] = dl * R;
    if (lane == 0) s_fabar = P;
  }
#pragma unroll
  for (int i = 0; i < VP; ++i) {
    const int t = tid + i * kBlock, j = t / VCH;
    if (j < F) *reinterpret_cast<uint4*>(&s_v[j * D + (t % VCH) * 8]) = vc[i];
  }
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    const int t = tid + i * kBlock, j = t / KCH;
    if (j < F) *reinterpret_cast<uint4*>(&s_k[j * N + (t % KCH) * 8]) = kc[i];
  }
  __syncthreads();
  float vj[RT][kVJ];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
    for (int m = 0; m < kVJ; ++m) {
      const int j = cq + 4 * m;
      vj[rt][m] = (j < F) ? bf16_to_f32(s_v[j * D + row]) : 0.f;
    }
  }
  if (F > 0) {
    settle_state<RT, NCT>(s);
    fold_and_store<D, N, RT, NCT, kVJ>(S0, s, s_fabar, s_k, s_fw, vj, F, wave, r, cq);
  }

  if (tid == 0) {
    if (h == 0) flag_error(p.err, bad);
    *reinterpret_cast<unsigned long long*>(rec + kMetaPtr) = pack_ptr((head + F) % L, 0, rp.pending);
  }
}

struct PtrParams {
  float* meta;
  int32_t* err;
  const int32_t* accepted;
  const int32_t* mask;
  const int32_t* slots;
  int rows;
  int B, H, L;
};

__device__ __forceinline__ unsigned long long* ptr_word(const PtrParams& p, int i) {
  return reinterpret_cast<unsigned long long*>(p.meta + (size_t)i * meta_words(p.L) + kMetaPtr);
}

// One thread per (request, head) record: count += clamp(accepted, 0, pending);
// pending = 0.
__global__ __launch_bounds__(kBlock) void rollback_kernel(PtrParams p) {
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i >= p.B * p.H) return;
  const int b = i / p.H, h = i - b * p.H;
  const int rb = pool_row(p.slots, p.rows, b, p.err, h == 0);
  if (rb < 0) return;
  unsigned long long* w = ptr_word(p, rb * p.H + h);
  const RingPtr rp = unpack_ptr(*w);
  int head = rp.head, cnt = rp.count, pend = rp.pending;
  int bad = 0;
  if (head >= p.L) {
    head %= p.L;
    bad |= RSSM_ERR_POINTERS;
  }
  commit_window(p.L, p.accepted[b], cnt, pend, bad);
  *w = pack_ptr(head, cnt, 0);
  flag_error(p.err, bad);
}

struct PtrViewParams {
  const float* meta;
  int32_t* err;
  int32_t* head;
  int32_t* count;
  int32_t* pending;
  const int32_t* slots;
  int rows;
  int B, H, L;
};

// One thread per (request, head) record, all loads independent: head 0's thread
// writes the fields of its pointer word as int32, every other head's thread
// compares its own word with head 0's.  (One thread per request looping over
// the H records took a memory round trip per record: 22 us at B = 256, H = 32.)
__global__ __launch_bounds__(kBlock) void ring_pointers_kernel(PtrViewParams p) {
  const long long i = (long long)blockIdx.x * kBlock + threadIdx.x;
  if (i >= (long long)p.B * p.H) return;
  const int b = (int)(i / p.H), h = (int)(i - (long long)b * p.H);
  const int rb = pool_row(p.slots, p.rows, b, p.err, h == 0);
  int hd = -1, ct = -1, pd = -1;
  if (rb >= 0) {
    const int MS = meta_words(p.L);
    const float* rec = p.meta + (size_t)rb * p.H * MS;
    const unsigned long long w0 = *reinterpret_cast<const unsigned long long*>(rec + kMetaPtr);
    if (h != 0) {
      const unsigned long long wh = *reinterpret_cast<const unsigned long long*>(rec + (size_t)h * MS + kMetaPtr);
      if (wh != w0) flag_error(p.err, RSSM_ERR_DIVERGED);
      return;
    }
    const RingPtr rp = unpack_ptr(w0);
    hd = rp.head;
    ct = rp.count;
    pd = rp.pending;
  } else if (h != 0) {
    return;
  }
  if (p.head != nullptr) p.head[b] = hd;
  if (p.count != nullptr) p.count[b] = ct;
  if (p.pending != nullptr) p.pending[b] = pd;
}

__global__ __launch_bounds__(kBlock) void ring_reset_kernel(PtrParams p) {
  const int i = blockIdx.x * kBlock + threadIdx.x;
  if (i == 0 && p.err != nullptr) *p.err = 0;
  if (i >= p.B * p.H) return;
  const int b = i / p.H, h = i - b * p.H;
  if (p.mask != nullptr && p.mask[b] == 0) return;
  const int rb = pool_row(p.slots, p.rows, b, nullptr, false);
  if (rb >= 0) *ptr_word(p, rb * p.H + h) = 0ull;
}

}  // namespace rssm

// ======================================================= C ABI
using namespace rssm;
using rssm_host::launch;

namespace {

ReplayParams make_replay_params(const rssm_dims* d, float* state0, rssm_ring* ring) {
  ReplayParams p{};
  p.state0 = state0;
  p.ring_v = static_cast<uint16_t*>(ring->vu);
  p.ring_k = ring->k;
  p.meta = reinterpret_cast<float*>(ring->meta);
  p.err = ring->err;
  p.slots = ring->slots;
  p.rows = ring->rows;
  p.y_bf16 = (d->flags & RSSM_F_Y_BF16) != 0;
  p.H = d->nheads;
  p.G = d->ngroups;
  p.L = d->capacity;
  return p;
}

}  // namespace

extern "C" int ssm_decode_step(const rssm_dims* dims, float* state, const uint16_t* v,
                               const uint16_t* k, const uint16_t* q, const float* dt,
                               const float* dt_bias, const float* A, float* y, void* stream) {
  if (!rssm_host::dims_ok(dims) || !state || !v || !k || !q || !dt || !dt_bias || !A || !y ||
      !rssm_host::aligned16(state, v, k, q, dt, dt_bias, A, y))
    return RSSM_EINVAL;
  if (!rssm_host::shape_supported(dims) || (dims->flags & RSSM_F_Y_BF16)) return RSSM_ENOTSUP;
  StdParams p{state, v, k, q, dt, dt_bias, A, y, dims->nheads, dims->ngroups};
  const dim3 grid(dims->batch * dims->nheads);
  const bool d64 = dims->head_dim == 64;
  switch (dims->state_dim) {
    case 64:
      return launch(d64 ? ssm_step_kernel<64, 64> : ssm_step_kernel<128, 64>, grid, dim3(kBlock), stream, p);
    case 256:
      return launch(d64 ? ssm_step_kernel<64, 256> : ssm_step_kernel<128, 256>, grid, dim3(kBlock), stream, p);
    default:
      return launch(d64 ? ssm_step_kernel<64, 128> : ssm_step_kernel<128, 128>, grid, dim3(kBlock), stream, p);
  }
}

extern "C" int replay_append_decode(const rssm_dims* dims, float* state0, rssm_ring* ring,
                                    const uint16_t* v, const uint16_t* k, const uint16_t* q,
                                    const float* dt, const float* dt_bias, const float* A,
                                    float* y, int32_t* flushed, void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::ring_ok(ring) || !state0 || !v || !k || !q ||
      !dt || !dt_bias || !A || !y || !rssm_host::aligned16(state0, v, k, q, dt, dt_bias, A, y, flushed))
    return RSSM_EINVAL;
  if (dims->capacity < 1) return RSSM_EINVAL;
  if (!rssm_host::ring_shape_supported(dims)) return RSSM_ENOTSUP;
  ReplayParams p = make_replay_params(dims, state0, ring);
  p.v = v;
  p.k = k;
  p.q = q;
  p.dt = dt;
  p.dt_bias = dt_bias;
  p.A = A;
  p.y = y;
  p.flushed = flushed;
  if (dims->state_dim == 64) return rssm_host::launch_replay_n64(0, dims->head_dim, p, dims->batch, stream);
  if (dims->state_dim == 256) return rssm_host::launch_replay_n256(0, dims->head_dim, p, dims->batch, stream);
  if (dims->head_dim == 64) return rssm_host::launch_window<64, 1, true>(p, dims->batch, stream);
  return rssm_host::launch_window<128, 1, true>(p, dims->batch, stream);
}

extern "C" int replay_append_decode_conv(const rssm_dims* dims, float* state0, rssm_ring* ring,
                                         const uint16_t* conv_state_in, uint16_t* conv_state_out,
                                         const uint16_t* xbc, const uint16_t* conv_w, const float* dt,
                                         const float* dt_bias, const float* A, float* y,
                                         int32_t* flushed, void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::ring_ok(ring) || !state0 || !conv_state_in ||
      !conv_state_out || !xbc || !conv_w || !dt || !dt_bias || !A || !y ||
      !rssm_host::aligned16(state0, conv_state_in, conv_state_out, xbc, conv_w, dt, dt_bias, A, y, flushed))
    return RSSM_EINVAL;
  if (conv_state_in == conv_state_out || dims->capacity < 1) return RSSM_EINVAL;
  if (!rssm_host::conv_shape_supported(dims)) return RSSM_ENOTSUP;
  ReplayParams p = make_replay_params(dims, state0, ring);
  p.conv_in = conv_state_in;
  p.conv_out = conv_state_out;
  p.xbc = xbc;
  p.conv_w = conv_w;
  p.dt = dt;
  p.dt_bias = dt_bias;
  p.A = A;
  p.y = y;
  p.flushed = flushed;
  if (dims->state_dim == 64) return rssm_host::launch_replay_conv_n64(dims->head_dim, p, dims->batch, stream);
  if (dims->state_dim == 256) return rssm_host::launch_replay_conv_n256(dims->head_dim, p, dims->batch, stream);
  if (dims->head_dim == 64) return rssm_host::launch_window<64, 1, true, true>(p, dims->batch, stream);
  return rssm_host::launch_window<128, 1, true, true>(p, dims->batch, stream);
}

namespace {

// the flush instances of one mode: EAGER when no mask selects the requests
template <bool EAGER>
int launch_replay_flush(const rssm_dims* dims, const ReplayParams& p, void* stream) {
  const dim3 grid(dims->batch * dims->nheads);
  const bool d64 = dims->head_dim == 64;
  switch (dims->state_dim) {
    case 64:
      return launch(d64 ? replay_flush_kernel<64, 64, EAGER> : replay_flush_kernel<128, 64, EAGER>, grid, dim3(kBlock),
                    stream, p);
    case 256:
      return launch(d64 ? replay_flush_kernel<64, 256, EAGER> : replay_flush_kernel<128, 256, EAGER>, grid, dim3(kBlock),
                    stream, p);
    default:
      return launch(d64 ? replay_flush_kernel<64, 128, EAGER> : replay_flush_kernel<128, 128, EAGER>, grid, dim3(kBlock),
                    stream, p);
  }
}

}  // namespace

extern "C" int replay_flush(const rssm_dims* dims, float* state0, rssm_ring* ring,
                            const int32_t* mask, void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::ring_ok(ring) || !state0 ||
      !rssm_host::aligned16(state0, mask))
    return RSSM_EINVAL;
  if (dims->capacity < 1) return RSSM_EINVAL;
  if (!rssm_host::ring_shape_supported(dims)) return RSSM_ENOTSUP;
  ReplayParams p = make_replay_params(dims, state0, ring);
  p.mask = mask;
  return mask == nullptr ? launch_replay_flush<true>(dims, p, stream) : launch_replay_flush<false>(dims, p, stream);
}

namespace {

int verify_common(const rssm_dims* dims, int32_t T, float* state0, rssm_ring* ring, const int32_t* accepted,
                  const uint16_t* v, const uint16_t* k, const uint16_t* q, const float* dt,
                  const float* dt_bias, const float* A, float* y, int32_t* flushed, void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::ring_ok(ring) || !state0 || !v || !k || !q ||
      !dt || !dt_bias || !A || !y || !rssm_host::aligned16(state0, v, k, q, dt, dt_bias, A, y, flushed))
    return RSSM_EINVAL;
  if (T < 1 || dims->capacity < 2 * T) return RSSM_EINVAL;
  if (!rssm_host::ring_shape_supported(dims) || T > kMaxT) return RSSM_ENOTSUP;
  ReplayParams p = make_replay_params(dims, state0, ring);
  p.accepted = accepted;
  p.v = v;
  p.k = k;
  p.q = q;
  p.dt = dt;
  p.dt_bias = dt_bias;
  p.A = A;
  p.y = y;
  p.flushed = flushed;
  const int D = dims->head_dim;
  if (dims->state_dim == 64) return rssm_host::launch_replay_n64(T, D, p, dims->batch, stream);
  if (dims->state_dim == 256) return rssm_host::launch_replay_n256(T, D, p, dims->batch, stream);
  if (T <= 4) return rssm_host::launch_replay_verify_lo(T, D, p, dims->batch, stream);
  return rssm_host::launch_replay_verify_hi(T, D, p, dims->batch, stream);
}

}  // namespace

extern "C" int replay_verify_T(const rssm_dims* dims, int32_t T, float* state0, rssm_ring* ring,
                               const uint16_t* v, const uint16_t* k, const uint16_t* q,
                               const float* dt, const float* dt_bias, const float* A, float* y,
                               int32_t* flushed, void* stream) {
  return verify_common(dims, T, state0, ring, nullptr, v, k, q, dt, dt_bias, A, y, flushed, stream);
}

extern "C" int replay_commit_verify_T(const rssm_dims* dims, int32_t T, float* state0, rssm_ring* ring,
                                      const int32_t* accepted, const uint16_t* v, const uint16_t* k,
                                      const uint16_t* q, const float* dt, const float* dt_bias,
                                      const float* A, float* y, int32_t* flushed, void* stream) {
  if (!accepted || !rssm_host::aligned16(accepted)) return RSSM_EINVAL;
  return verify_common(dims, T, state0, ring, accepted, v, k, q, dt, dt_bias, A, y, flushed, stream);
}

extern "C" int replay_rollback(const rssm_dims* dims, rssm_ring* ring, const int32_t* accepted,
                               void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::meta_ok(ring) || !accepted || !rssm_host::aligned16(accepted))
    return RSSM_EINVAL;
  if (dims->capacity < 1) return RSSM_EINVAL;
  if (dims->capacity > kMaxL) return RSSM_ENOTSUP;
  PtrParams p{reinterpret_cast<float*>(ring->meta), ring->err, accepted, nullptr, ring->slots, ring->rows,
              dims->batch, dims->nheads, dims->capacity};
  const dim3 grid((dims->batch * dims->nheads + kBlock - 1) / kBlock);
  return launch(rollback_kernel, grid, dim3(kBlock), stream, p);
}

extern "C" int rssm_ring_reset(const rssm_dims* dims, rssm_ring* ring, const int32_t* mask,
                               void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::meta_ok(ring) || !rssm_host::aligned16(mask)) return RSSM_EINVAL;
  if (dims->capacity < 1) return RSSM_EINVAL;
  if (dims->capacity > kMaxL) return RSSM_ENOTSUP;
  PtrParams p{reinterpret_cast<float*>(ring->meta), ring->err, nullptr, mask, ring->slots, ring->rows,
              dims->batch, dims->nheads, dims->capacity};
  const dim3 grid((dims->batch * dims->nheads + kBlock - 1) / kBlock);
  return launch(ring_reset_kernel, grid, dim3(kBlock), stream, p);
}

extern "C" int rssm_ring_pointers(const rssm_dims* dims, const rssm_ring* ring, int32_t* head,
                                  int32_t* count, int32_t* pending, void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::meta_ok(ring) || !rssm_host::aligned16(head, count, pending))
    return RSSM_EINVAL;
  if (dims->capacity < 1) return RSSM_EINVAL;
  if (dims->capacity > kMaxL) return RSSM_ENOTSUP;
  PtrViewParams p{reinterpret_cast<const float*>(ring->meta), ring->err, head, count, pending, ring->slots,
                  ring->rows, dims->batch, dims->nheads, dims->capacity};
  const dim3 grid((unsigned)(((long long)dims->batch * dims->nheads + kBlock - 1) / kBlock));
  return launch(ring_pointers_kernel, grid, dim3(kBlock), stream, p);
}
