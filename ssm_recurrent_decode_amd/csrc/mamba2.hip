// Mamba-2 decode kernels for gfx950: the standard step with state write-back, and
// ReplaySSM append-decode / speculative verify / flush / rollback.
//
// Method: "ReplaySSM: Cache SSM Inputs, Not State" -- background (the recurrence),
// method (core idea, output-only decode, rollback as a pointer move), algorithms
// (Mamba-2 standard decode; speculative decoding with the early-flush rule) and
// kernel design (shared inner products, ring indexed in-kernel).
//
// Work decomposition: one work-group of four waves per (request b, head h).  Each
// wave streams D/64 row tiles of the head's d x n fp32 state in the tile layout
// described in common.hpp (one float4 per lane per 16x16 tile, all loads issued
// before any dependent arithmetic).  Work-groups are renumbered so that the heads
// of a request land on one XCD.
#include "common.hpp"

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
  float4 s[RT][NCT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) s[rt][ct] = ld_f4(S + row * N + ct * 16 + cq * 4);
  }
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
    for (int ct = 0; ct < NCT; ++ct) {
      float4 x = s[rt][ct];
      x.x = a * x.x + dv * bf16_lo(kk[ct].x);
      x.y = a * x.y + dv * bf16_hi(kk[ct].x);
      x.z = a * x.z + dv * bf16_lo(kk[ct].y);
      x.w = a * x.w + dv * bf16_hi(kk[ct].y);
      acc += dot4_bf16(x, qq[ct]);
      st_f4(S + row * N + ct * 16 + cq * 4, x);
    }
    acc = reduce_row4(acc);
    if (cq == 0) p.y[(size_t)wg * D + row] = acc;
  }
}

// ======================================================= ReplaySSM
struct ReplayParams {
  float* state0;
  uint16_t* ring_v;
  uint16_t* ring_k;
  float* ring_dt;
  float* ring_decay;
  int32_t* head;
  int32_t* count;
  int32_t* pending;
  int32_t* arrive;
  int32_t* err;
  const uint16_t* v;   // [B, T, H, D]
  const uint16_t* k;   // [B, T, G, N]
  const uint16_t* q;   // [B, T, G, N]
  const float* dt;     // [B, T, H]
  const float* dt_bias;
  const float* A;
  float* y;            // [B, T, H, D]
  int32_t* flushed;
  const int32_t* mask;  // explicit flush only
  int H, G, L;
};

// One kernel for both decode modes.
//  APPEND (T == 1): append the token; it is entry c of E = c + 1; flush all E
//    entries when E == L (flush-when-full).  count <- E or 0.
//  VERIFY (T drafts): drafts are entries c .. c+T-1; draft s reads p_s = c+s+1
//    entries; if c + 2T > L fold the c committed entries only.  pending <- T.
// Every global load is issued unconditionally with clamped indices (results are
// selected afterwards), so the loads of a work-group go out back to back and the
// first wait comes at the first use.
template <int D, int N, int T, bool APPEND>
__global__ __launch_bounds__(kBlock) void replay_window_kernel(ReplayParams p) {
  static_assert(N == 128, "key/query staging assumes n = 128 (16 lanes x 8 values)");
  constexpr int NCT = N / 16;
  constexpr int RT = D / (16 * kWavesPerBlock);
  __shared__ float s_w[T][kMaxL];     // w_{j,s}, zero where j >= p_s
  __shared__ float s_M[T][kMaxL];     // k_j . q_s
  __shared__ float s_abar[T];
  __shared__ float s_fw[kMaxL];
  __shared__ float s_fabar;
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kMaxL * N];

  const int H = p.H, G = p.G, L = p.L;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int b = wg / H, h = wg - b * H, hpg = H / G, g = h / hpg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, cq = lane >> 4;
  const size_t bh = (size_t)b * H + h;
  float* S0 = p.state0 + bh * D * N;

  // ---- checkpoint tiles first: their addresses need no ring pointer
  float4 s[RT][NCT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) s[rt][ct] = ld_f4(S0 + row * N + ct * 16 + cq * 4);
  }
  uint2 qt[T][NCT];
#pragma unroll
  for (int sd = 0; sd < T; ++sd) {
    const uint16_t* qp = p.q + (((size_t)b * T + sd) * G + g) * N + cq * 4;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) qt[sd][ct] = ld_u2(qp + ct * 16);
  }

  // ---- ring pointers (uniform per request), clamped into range
  int head = p.head[b], cnt = p.count[b];
  const int pend = p.pending[b];
  int bad = 0;
  if (head < 0 || head >= L) {
    head = ((head % L) + L) % L;
    bad |= RSSM_ERR_POINTERS;
  }
  const int cmax = APPEND ? L - 1 : L - T;
  if (cnt < 0 || cnt > cmax) {
    cnt = cnt < 0 ? 0 : cmax;
    bad |= RSSM_ERR_POINTERS;
  }
  if (pend != 0) bad |= RSSM_ERR_PENDING;
  const int c = cnt;
  const int E = c + T;
  const bool do_flush = APPEND ? (E == L) : (c + 2 * T > L);
  const int F = do_flush ? (APPEND ? E : c) : 0;
  const bool write_new = !(APPEND && do_flush);
  int arrival = 0;
  if (tid == 0) arrival = arrive_after_reading(&p.arrive[b], head, cnt, pend);

  // ---- v_j[row] of the entries this lane combines (j = cq + 4m)
  float vj[RT][kVJ];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
    for (int m = 0; m < kVJ; ++m) {
      const int j = cq + 4 * m;
      const int jj = min(j, E - 1);
      const uint16_t* src = (jj < c) ? p.ring_v + (bh * L + ring_slot(head, jj, L)) * D
                                     : p.v + (((size_t)b * T + max(jj - c, 0)) * H + h) * D;
      const float val = bf16_to_f32(src[row]);
      vj[rt][m] = (j < E) ? val : 0.f;
    }
  }

  // ---- keys and queries for the shared inner products M_{j,s} = k_j . q_s
  //      (16 lanes per entry, 8 columns each; passes of 16 entries per block)
  const int sub = lane & 15;
  uint4 qm[T];
#pragma unroll
  for (int sd = 0; sd < T; ++sd) qm[sd] = ld_u4(p.q + (((size_t)b * T + sd) * G + g) * N + sub * 8);
  constexpr int kPasses = kMaxL / 16;
  uint4 kj[kPasses];
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    const int j = ps * 16 + wave * 4 + (lane >> 4);
    const int jj = min(j, E - 1);
    const uint16_t* src = (jj < c)
        ? p.ring_k + (((size_t)b * G + g) * L + ring_slot(head, jj, L)) * N
        : p.k + (((size_t)b * T + max(jj - c, 0)) * G + g) * N;
    kj[ps] = ld_u4(src + sub * 8);
  }

  // ---- wave 0: step sizes and decays of all entries, then every weight by
  //      suffix-product scans (one per draft boundary, one for the fold)
  if (wave == 0) {
    const int j = lane;
    const int jj = min(j, E - 1);
    const size_t o = bh * L + ring_slot(head, max(min(jj, c - 1), 0), L);
    const float dl_ring = p.ring_dt[o], al_ring = p.ring_decay[o];
    const int sdj = max(jj - c, 0);
    const float dl_new = softplus_f32(p.dt[((size_t)b * T + sdj) * H + h] + p.dt_bias[h]);
    const float al_new = expf(p.A[h] * dl_new);
    const bool valid = j < E, cached = jj < c;
    const float dl = valid ? (cached ? dl_ring : dl_new) : 0.f;
    const float al = valid ? (cached ? al_ring : al_new) : 1.f;
#pragma unroll
    for (int sd = 0; sd < T; ++sd) {
      const int m = c + sd;  // last entry seen by draft sd
      float all;
      const float ex = suffix_product_excl(j <= m ? al : 1.f, lane, &all);
      if (j < kMaxL) s_w[sd][j] = (j <= m) ? dl * ex : 0.f;
      if (lane == 0) s_abar[sd] = all;
    }
    {
      float all;
      const float ex = suffix_product_excl(j < F ? al : 1.f, lane, &all);
      if (j < kMaxL) s_fw[j] = (j < F) ? dl * ex : 0.f;
      if (lane == 0) s_fabar = all;
    }
    if (write_new && j >= c && j < E) {  // cache the new entries' step size and decay
      const size_t on = bh * L + ring_slot(head, j, L);
      p.ring_dt[on] = dl;
      p.ring_decay[on] = al;
    }
  }

  // ---- all waves: inner products and staging of the keys to fold
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    const int j = ps * 16 + wave * 4 + (lane >> 4);
    const uint4 kv = (j < E) ? kj[ps] : make_uint4(0, 0, 0, 0);
    if (j < F) *reinterpret_cast<uint4*>(&s_k[j * N + sub * 8]) = kv;
#pragma unroll
    for (int sd = 0; sd < T; ++sd) {
      const float dv = reduce_quarter(dot8_bf16(kv, qm[sd]));
      if (sub == 0 && j < kMaxL) s_M[sd][j] = dv;
    }
  }
  __syncthreads();

  // ---- output-only route: y_s = abar_s (S_0 q_s) + sum_j w_{j,s} M_{j,s} v_j
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
    float dots[T];
#pragma unroll
    for (int sd = 0; sd < T; ++sd) dots[sd] = 0.f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int sd = 0; sd < T; ++sd) dots[sd] += dot4_bf16(s[rt][ct], qt[sd][ct]);
#pragma unroll
    for (int sd = 0; sd < T; ++sd) {
      float part = s_abar[sd] * dots[sd];
#pragma unroll
      for (int m = 0; m < kVJ; ++m) {
        const int j = cq + 4 * m;
        part += s_w[sd][j] * s_M[sd][j] * vj[rt][m];  // both zero beyond p_s
      }
      part = reduce_row4(part);
      if ((sd & 3) == cq) p.y[(((size_t)b * T + sd) * H + h) * D + row] = part;
    }
  }

  // ---- fused flush (per-request runtime decision)
  if (F > 0) fold_and_store<D, N, RT, NCT>(S0, s, s_fabar, s_k, s_fw, vj, F, wave, r, cq);

  // ---- cache the new entries' v (this head) and k (group owner head only)
  if (write_new) {
    for (int t = tid; t < T * (D / 8); t += kBlock) {
      const int sd = t / (D / 8), o = (t % (D / 8)) * 8;
      const size_t slot = ring_slot(head, c + sd, L);
      *reinterpret_cast<uint4*>(p.ring_v + (bh * L + slot) * D + o) =
          ld_u4(p.v + (((size_t)b * T + sd) * H + h) * D + o);
    }
    if (h % hpg == 0) {
      for (int t = tid; t < T * (N / 8); t += kBlock) {
        const int sd = t / (N / 8), o = (t % (N / 8)) * 8;
        const size_t slot = ring_slot(head, c + sd, L);
        *reinterpret_cast<uint4*>(p.ring_k + (((size_t)b * G + g) * L + slot) * N + o) =
            ld_u4(p.k + (((size_t)b * T + sd) * G + g) * N + o);
      }
    }
  }

  // ---- pointer update by the last work-group of the request to read them
  if (tid == 0) {
    if (h == 0) {
      flag_error(p.err, bad);
      if (p.flushed != nullptr) p.flushed[b] = do_flush ? 1 : 0;
    }
    if (arrival == H - 1) {
      p.arrive[b] = 0;
      if (APPEND) {
        p.head[b] = do_flush ? ring_slot(head, E % L, L) : head;
        p.count[b] = do_flush ? 0 : E;
        p.pending[b] = 0;
      } else {
        p.head[b] = do_flush ? ring_slot(head, c % L, L) : head;
        p.count[b] = do_flush ? 0 : c;
        p.pending[b] = T;
      }
    }
  }
}

// Explicit flush of the committed entries of masked requests.
template <int D, int N>
__global__ __launch_bounds__(kBlock) void replay_flush_kernel(ReplayParams p) {
  constexpr int NCT = N / 16;
  constexpr int RT = D / (16 * kWavesPerBlock);
  __shared__ float s_fw[kMaxL];
  __shared__ float s_fabar;
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kMaxL * N];

  const int H = p.H, G = p.G, L = p.L;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int b = wg / H, h = wg - b * H, g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, cq = lane >> 4;

  if (p.mask != nullptr && p.mask[b] == 0) return;
  int head = p.head[b], cnt = p.count[b];
  const int pend = p.pending[b];
  int bad = 0;
  if (head < 0 || head >= L) {
    head = ((head % L) + L) % L;
    bad |= RSSM_ERR_POINTERS;
  }
  if (cnt < 0 || cnt > L) {
    cnt = cnt < 0 ? 0 : L;
    bad |= RSSM_ERR_POINTERS;
  }
  if (pend < 0 || cnt + pend > L) bad |= RSSM_ERR_POINTERS;
  if (cnt == 0) {
    if (h == 0 && tid == 0) flag_error(p.err, bad);
    return;
  }
  const int F = cnt;
  const size_t bh = (size_t)b * H + h;
  float* S0 = p.state0 + bh * D * N;

  float4 s[RT][NCT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) s[rt][ct] = ld_f4(S0 + row * N + ct * 16 + cq * 4);
  }
  int arrival = 0;
  if (tid == 0) arrival = arrive_after_reading(&p.arrive[b], head, cnt, pend);
  float vj[RT][kVJ];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
    for (int m = 0; m < kVJ; ++m) {
      const int j = cq + 4 * m;
      vj[rt][m] = (j < F) ? bf16_to_f32(p.ring_v[(bh * L + (head + j) % L) * D + row]) : 0.f;
    }
  }
  if (wave == 0) {
    const int j = lane;
    float dl = 0.f, al = 1.f;
    if (j < F) {
      const size_t o = bh * L + (head + j) % L;
      dl = p.ring_dt[o];
      al = p.ring_decay[o];
    }
    float R = 1.f, P = 1.f;
    for (int m = 0; m < F; ++m) {
      const float am = __shfl(al, m, kWave);
      P *= am;
      if (m > j) R *= am;
    }
    if (j < F) s_fw[j] = dl * R;
    if (lane == 0) s_fabar = P;
  }
  for (int t = tid; t < F * (N / 8); t += kBlock) {
    const int j = t / (N / 8), o = (t % (N / 8)) * 8;
    *reinterpret_cast<uint4*>(&s_k[j * N + o]) =
        ld_u4(p.ring_k + (((size_t)b * G + g) * L + (head + j) % L) * N + o);
  }
  __syncthreads();
  fold_and_store<D, N, RT, NCT>(S0, s, s_fabar, s_k, s_fw, vj, F, wave, r, cq);

  if (tid == 0) {
    if (h == 0) flag_error(p.err, bad);
    if (arrival == H - 1) {
      p.arrive[b] = 0;
      p.head[b] = (head + F) % L;
      p.count[b] = 0;
    }
  }
}

struct PtrParams {
  int32_t* head;
  int32_t* count;
  int32_t* pending;
  int32_t* err;
  const int32_t* accepted;
  const int32_t* mask;
  int B, L;
};

// count += clamp(accepted, 0, pending); pending = 0.
__global__ __launch_bounds__(kBlock) void rollback_kernel(PtrParams p) {
  const int b = blockIdx.x * kBlock + threadIdx.x;
  if (b >= p.B) return;
  int cnt = p.count[b], pend = p.pending[b], acc = p.accepted[b];
  int bad = 0;
  if (pend < 0 || pend > p.L) {
    pend = pend < 0 ? 0 : p.L;
    bad |= RSSM_ERR_POINTERS;
  }
  if (cnt < 0 || cnt + pend > p.L) {
    cnt = cnt < 0 ? 0 : (p.L - pend < 0 ? 0 : p.L - pend);
    bad |= RSSM_ERR_POINTERS;
  }
  if (acc < 0 || acc > pend) {
    acc = acc < 0 ? 0 : pend;
    bad |= RSSM_ERR_ACCEPTED;
  }
  p.count[b] = cnt + acc;
  p.pending[b] = 0;
  flag_error(p.err, bad);
}

__global__ __launch_bounds__(kBlock) void ring_reset_kernel(PtrParams p) {
  const int b = blockIdx.x * kBlock + threadIdx.x;
  if (b == 0 && p.err != nullptr) *p.err = 0;
  if (b >= p.B) return;
  if (p.mask == nullptr || p.mask[b] != 0) {
    p.head[b] = 0;
    p.count[b] = 0;
    p.pending[b] = 0;
  }
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
  p.ring_dt = ring->dt;
  p.ring_decay = ring->decay;
  p.head = ring->head;
  p.count = ring->count;
  p.pending = ring->pending;
  p.arrive = ring->arrive;
  p.err = ring->err;
  p.H = d->nheads;
  p.G = d->ngroups;
  p.L = d->capacity;
  return p;
}

template <int T>
int launch_verify(int D, const ReplayParams& p, dim3 grid, void* stream) {
  if (D == 64) return launch(replay_window_kernel<64, 128, T, false>, grid, dim3(kBlock), stream, p);
  return launch(replay_window_kernel<128, 128, T, false>, grid, dim3(kBlock), stream, p);
}

}  // namespace

extern "C" int ssm_decode_step(const rssm_dims* dims, float* state, const uint16_t* v,
                               const uint16_t* k, const uint16_t* q, const float* dt,
                               const float* dt_bias, const float* A, float* y, void* stream) {
  if (!rssm_host::dims_ok(dims) || !state || !v || !k || !q || !dt || !dt_bias || !A || !y)
    return RSSM_EINVAL;
  if (!rssm_host::shape_supported(dims)) return RSSM_ENOTSUP;
  StdParams p{state, v, k, q, dt, dt_bias, A, y, dims->nheads, dims->ngroups};
  const dim3 grid(dims->batch * dims->nheads);
  if (dims->head_dim == 64) return launch(ssm_step_kernel<64, 128>, grid, dim3(kBlock), stream, p);
  return launch(ssm_step_kernel<128, 128>, grid, dim3(kBlock), stream, p);
}

extern "C" int replay_append_decode(const rssm_dims* dims, float* state0, rssm_ring* ring,
                                    const uint16_t* v, const uint16_t* k, const uint16_t* q,
                                    const float* dt, const float* dt_bias, const float* A,
                                    float* y, int32_t* flushed, void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::ring_ok(ring, true) || !state0 || !v || !k || !q ||
      !dt || !dt_bias || !A || !y)
    return RSSM_EINVAL;
  if (dims->capacity < 1) return RSSM_EINVAL;
  if (!rssm_host::shape_supported(dims) || dims->capacity > kMaxL) return RSSM_ENOTSUP;
  ReplayParams p = make_replay_params(dims, state0, ring);
  p.v = v;
  p.k = k;
  p.q = q;
  p.dt = dt;
  p.dt_bias = dt_bias;
  p.A = A;
  p.y = y;
  p.flushed = flushed;
  const dim3 grid(dims->batch * dims->nheads);
  if (dims->head_dim == 64)
    return launch(replay_window_kernel<64, 128, 1, true>, grid, dim3(kBlock), stream, p);
  return launch(replay_window_kernel<128, 128, 1, true>, grid, dim3(kBlock), stream, p);
}

extern "C" int replay_flush(const rssm_dims* dims, float* state0, rssm_ring* ring,
                            const int32_t* mask, void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::ring_ok(ring, true) || !state0) return RSSM_EINVAL;
  if (dims->capacity < 1) return RSSM_EINVAL;
  if (!rssm_host::shape_supported(dims) || dims->capacity > kMaxL) return RSSM_ENOTSUP;
  ReplayParams p = make_replay_params(dims, state0, ring);
  p.mask = mask;
  const dim3 grid(dims->batch * dims->nheads);
  if (dims->head_dim == 64) return launch(replay_flush_kernel<64, 128>, grid, dim3(kBlock), stream, p);
  return launch(replay_flush_kernel<128, 128>, grid, dim3(kBlock), stream, p);
}

extern "C" int replay_verify_T(const rssm_dims* dims, int32_t T, float* state0, rssm_ring* ring,
                               const uint16_t* v, const uint16_t* k, const uint16_t* q,
                               const float* dt, const float* dt_bias, const float* A, float* y,
                               int32_t* flushed, void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::ring_ok(ring, true) || !state0 || !v || !k || !q ||
      !dt || !dt_bias || !A || !y)
    return RSSM_EINVAL;
  if (T < 1 || dims->capacity < 2 * T) return RSSM_EINVAL;
  if (!rssm_host::shape_supported(dims) || dims->capacity > kMaxL || T > kMaxT) return RSSM_ENOTSUP;
  ReplayParams p = make_replay_params(dims, state0, ring);
  p.v = v;
  p.k = k;
  p.q = q;
  p.dt = dt;
  p.dt_bias = dt_bias;
  p.A = A;
  p.y = y;
  p.flushed = flushed;
  const dim3 grid(dims->batch * dims->nheads);
  const int D = dims->head_dim;
  switch (T) {
    case 1: return launch_verify<1>(D, p, grid, stream);
    case 2: return launch_verify<2>(D, p, grid, stream);
    case 3: return launch_verify<3>(D, p, grid, stream);
    case 4: return launch_verify<4>(D, p, grid, stream);
    case 5: return launch_verify<5>(D, p, grid, stream);
    case 6: return launch_verify<6>(D, p, grid, stream);
    case 7: return launch_verify<7>(D, p, grid, stream);
    default: return launch_verify<8>(D, p, grid, stream);
  }
}

extern "C" int replay_rollback(const rssm_dims* dims, rssm_ring* ring, const int32_t* accepted,
                               void* stream) {
  if (!rssm_host::dims_ok(dims) || ring == nullptr || !ring->count || !ring->pending || !accepted)
    return RSSM_EINVAL;
  if (dims->capacity < 1) return RSSM_EINVAL;
  PtrParams p{ring->head, ring->count, ring->pending, ring->err, accepted, nullptr,
              dims->batch, dims->capacity};
  const dim3 grid((dims->batch + kBlock - 1) / kBlock);
  return launch(rollback_kernel, grid, dim3(kBlock), stream, p);
}

extern "C" int rssm_ring_reset(const rssm_dims* dims, rssm_ring* ring, const int32_t* mask,
                               void* stream) {
  if (!rssm_host::dims_ok(dims) || ring == nullptr || !ring->head || !ring->count || !ring->pending)
    return RSSM_EINVAL;
  PtrParams p{ring->head, ring->count, ring->pending, ring->err, nullptr, mask, dims->batch,
              dims->capacity};
  const dim3 grid((dims->batch + kBlock - 1) / kBlock);
  return launch(ring_reset_kernel, grid, dim3(kBlock), stream, p);
}
