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
// in the tile layout of common.hpp.  In the verify kernel the 2T readouts
// S_0 [k_1..k_T, q_1..q_T] run on the matrix cores straight from the state
// registers, and the per-row correction/solve/output runs one thread per row.
#include "common.hpp"

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
  const float alpha = expf(p.g[wg]);
  const float beta = p.beta[wg];

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
    float sk = 0.f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) sk += dot4_bf16(s[rt][ct], kk[ct]);
    sk = reduce_row4(sk);
    const float u = beta * (vr[rt] - alpha * sk);
    float acc = 0.f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float4 x = s[rt][ct];
      x.x = alpha * x.x + u * bf16_lo(kk[ct].x);
      x.y = alpha * x.y + u * bf16_hi(kk[ct].x);
      x.z = alpha * x.z + u * bf16_lo(kk[ct].y);
      x.w = alpha * x.w + u * bf16_hi(kk[ct].y);
      acc += dot4_bf16(x, qq[ct]);
      st_f4(S + row * N + ct * 16 + cq * 4, x);
    }
    acc = reduce_row4(acc);
    if (cq == 0) p.y[(size_t)wg * D + row] = acc;
  }
}

// ======================================================= ReplaySSM GDN
struct GdnReplayParams {
  float* state0;
  float* ring_u;       // [B, H, L, D] fp32
  uint16_t* ring_k;    // [B, G, L, N]
  float* ring_alpha;   // [B, H, L]
  unsigned long long* ptr;  // [B, H] packed ring pointer words, one copy per head
  int32_t* err;
  const uint16_t* v;   // [B, T, H, D]
  const uint16_t* k;   // [B, T, G, N]
  const uint16_t* q;   // [B, T, G, N]
  const float* g;      // [B, T, H]
  const float* beta;   // [B, T, H]
  float* y;            // [B, T, H, D]
  int32_t* flushed;
  const int32_t* mask;
  int H, G, L;
};

template <int D, int N, int T>
__global__ __launch_bounds__(kBlock) void gdn_verify_kernel(GdnReplayParams p) {
  static_assert(N == 128, "key staging assumes n = 128");
  static_assert(2 * T <= 16, "readout vectors must fit one MFMA M axis");
  static_assert(D <= kBlock, "one thread per state row in the solve");
  constexpr int NCT = N / 16;
  constexpr int RT = D / (16 * kWavesPerBlock);
  constexpr int NV = 2 * T;           // readout vectors: k_0..k_{T-1}, q_0..q_{T-1}
  __shared__ float s_Z[NV][D];        // (S_0 x_v)[row]
  __shared__ float s_M[NV][kMaxL];    // k_j . x_v, entries j < E (committed, then drafts)
  __shared__ float s_w[kMaxL];        // w_j = prod_{j<i<c} alpha_i  (committed j < c)
  __shared__ float s_abar;            // prod_{i<c} alpha_i
  __shared__ float s_alpha_d[T];      // draft decays
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kMaxL * N];

  const int H = p.H, G = p.G, L = p.L;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int b = wg / H, h = wg - b * H, hpg = H / G, g = h / hpg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, cq = lane >> 4;

  // ---- this head's copy of the pointer word and the checkpoint tiles, which
  //      need no pointer, in flight together
  const size_t bh = (size_t)b * H + h;
  const unsigned long long word = p.ptr[bh];
  float* S0 = p.state0 + bh * D * N;
  float4 s[RT][NCT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) s[rt][ct] = ld_f4(S0 + row * N + ct * 16 + cq * 4);
  }
  const RingPtr rp = unpack_ptr(word);
  int head = rp.head, cnt = rp.count;
  int bad = 0;
  if (head >= L) {
    head %= L;
    bad |= RSSM_ERR_POINTERS;
  }
  if (cnt > L - T) {
    cnt = L - T;
    bad |= RSSM_ERR_POINTERS;
  }
  if (rp.pending != 0) bad |= RSSM_ERR_PENDING;
  const int c = cnt;
  const int E = c + T;
  const bool do_flush = (c + 2 * T > L);
  const int F = do_flush ? c : 0;

  // ---- long-latency loads: this lane's readout vector at the tile columns;
  //      per-row ring corrections; fold operands
  uint2 xv[NCT];
  {
    const int vsel = r;  // MFMA M index = readout vector
    const uint16_t* src = nullptr;
    if (vsel < T) src = p.k + (((size_t)b * T + vsel) * G + g) * N;
    else if (vsel < NV) src = p.q + (((size_t)b * T + (vsel - T)) * G + g) * N;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) xv[ct] = src ? ld_u2(src + ct * 16 + cq * 4) : make_uint2(0, 0);
  }
  const int rho = tid;  // solve row
  float uj[kMaxL];
  float vd[T];
#pragma unroll
  for (int j = 0; j < kMaxL; ++j)
    uj[j] = (rho < D && j < c) ? p.ring_u[(bh * L + (head + j) % L) * D + rho] : 0.f;
#pragma unroll
  for (int sd = 0; sd < T; ++sd)
    vd[sd] = (rho < D) ? bf16_to_f32(p.v[(((size_t)b * T + sd) * H + h) * D + rho]) : 0.f;
  float uf[RT][kVJ];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
    for (int m = 0; m < kVJ; ++m) {
      const int j = cq + 4 * m;
      uf[rt][m] = (j < F) ? p.ring_u[(bh * L + (head + j) % L) * D + row] : 0.f;
    }
  }

  // ---- wave 0: decays of the committed entries and of the drafts
  if (wave == 0) {
    const int j = lane;
    float al = 1.f;
    if (j < c) al = p.ring_alpha[bh * L + (head + j) % L];
    else if (j < E) al = expf(p.g[((size_t)b * T + (j - c)) * H + h]);
    float R = 1.f, P = 1.f;
    for (int m = 0; m < c; ++m) {
      const float am = __shfl(al, m, kWave);
      P *= am;
      if (m > j) R *= am;
    }
    if (j < c) s_w[j] = R;
    if (j >= c && j < E) {
      s_alpha_d[j - c] = al;
      p.ring_alpha[bh * L + (head + j) % L] = al;
    }
    if (lane == 0) s_abar = P;
  }

  // ---- all waves: k_j . x_v for every entry (16 lanes per entry); stage keys to fold
  {
    const int sub = lane & 15;
    uint4 xm[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const uint16_t* src = (v < T) ? p.k + (((size_t)b * T + v) * G + g) * N
                                    : p.q + (((size_t)b * T + (v - T)) * G + g) * N;
      xm[v] = ld_u4(src + sub * 8);
    }
    for (int e0 = wave * 4; e0 < E; e0 += 16) {
      const int j = e0 + (lane >> 4);
      uint4 kj = make_uint4(0, 0, 0, 0);
      if (j < E) {
        const uint16_t* src =
            (j < c) ? p.ring_k + (((size_t)b * G + g) * L + (head + j) % L) * N
                    : p.k + (((size_t)b * T + (j - c)) * G + g) * N;
        kj = ld_u4(src + sub * 8);
        if (j < F) *reinterpret_cast<uint4*>(&s_k[j * N + sub * 8]) = kj;
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const float d = reduce_quarter(dot8_bf16(kj, xm[v]));
        if (sub == 0 && j < E) s_M[v][j] = d;
      }
    }
  }

  // ---- readouts Z = S_0 [K|Q] on the matrix cores: A[m][k] = x_m[col], B[k][nn] =
  //      S_0[row nn][col]; lane (r, cq) ends with Z[4cq+i][row r of the tile]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      acc = mfma4(bf16_lo(xv[ct].x), s[rt][ct].x, acc);
      acc = mfma4(bf16_hi(xv[ct].x), s[rt][ct].y, acc);
      acc = mfma4(bf16_lo(xv[ct].y), s[rt][ct].z, acc);
      acc = mfma4(bf16_hi(xv[ct].y), s[rt][ct].w, acc);
    }
    const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * cq + i < NV) s_Z[4 * cq + i][row] = acc[i];
  }
  __syncthreads();

  // ---- per row: committed-state readouts, corrections by forward substitution,
  //      outputs, and the corrections cached in the ring
  if (rho < D) {
    const float abar = s_abar;
    float sh[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      float acc = abar * s_Z[v][rho];
#pragma unroll
      for (int j = 0; j < kMaxL; ++j)
        if (j < c) acc += s_w[j] * uj[j] * s_M[v][j];
      sh[v] = acc;  // (S_h x_v)[rho]
    }
    float gamma[T];
    {
      float gm = 1.f;
#pragma unroll
      for (int sd = 0; sd < T; ++sd) {
        gm *= s_alpha_d[sd];
        gamma[sd] = gm;
      }
    }
    float u[T];
#pragma unroll
    for (int sd = 0; sd < T; ++sd) {
      const float bt = p.beta[((size_t)b * T + sd) * H + h];
      float acc = bt * (vd[sd] - gamma[sd] * sh[sd]);  // R_s
      float ratio = 1.f;                               // prod_{s'<i<=s} alpha_i
#pragma unroll
      for (int sp = sd - 1; sp >= 0; --sp) {
        ratio *= s_alpha_d[sp + 1];
        acc -= bt * ratio * s_M[sd][c + sp] * u[sp];  // A_{s,s'} u_{s'}
      }
      u[sd] = acc;
    }
#pragma unroll
    for (int sd = 0; sd < T; ++sd) {
      float acc = gamma[sd] * sh[T + sd];
      float ratio = 1.f;
#pragma unroll
      for (int sp = sd; sp >= 0; --sp) {
        if (sp < sd) ratio *= s_alpha_d[sp + 1];
        acc += ratio * s_M[T + sd][c + sp] * u[sp];
      }
      p.y[(((size_t)b * T + sd) * H + h) * D + rho] = acc;
      p.ring_u[(bh * L + (head + c + sd) % L) * D + rho] = u[sd];
    }
  }

  // ---- early flush of the committed entries
  if (F > 0) fold_and_store<D, N, RT, NCT, kVJ>(S0, s, s_abar, s_k, s_w, uf, F, wave, r, cq);

  // ---- draft keys cached by the group's owner head
  if (h % hpg == 0) {
    for (int t = tid; t < T * (N / 8); t += kBlock) {
      const int sd = t / (N / 8), o = (t % (N / 8)) * 8;
      const size_t slot = (head + c + sd) % L;
      *reinterpret_cast<uint4*>(p.ring_k + (((size_t)b * G + g) * L + slot) * N + o) =
          ld_u4(p.k + (((size_t)b * T + sd) * G + g) * N + o);
    }
  }

  if (tid == 0) {
    if (h == 0) {
      flag_error(p.err, bad);
      if (p.flushed != nullptr) p.flushed[b] = do_flush ? 1 : 0;
    }
    p.ptr[bh] = pack_ptr(do_flush ? (head + c) % L : head, do_flush ? 0 : c, T);
  }
}

// Explicit GDN flush of the committed entries of masked requests.
template <int D, int N>
__global__ __launch_bounds__(kBlock) void gdn_flush_kernel(GdnReplayParams p) {
  constexpr int NCT = N / 16;
  constexpr int RT = D / (16 * kWavesPerBlock);
  __shared__ float s_w[kMaxL];
  __shared__ float s_abar;
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kMaxL * N];

  const int H = p.H, G = p.G, L = p.L;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int b = wg / H, h = wg - b * H, g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, cq = lane >> 4;

  if (p.mask != nullptr && p.mask[b] == 0) return;
  const size_t bh = (size_t)b * H + h;
  const RingPtr rp = unpack_ptr(p.ptr[bh]);
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
  float* S0 = p.state0 + bh * D * N;
  float4 s[RT][NCT];
  if (F > 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) s[rt][ct] = ld_f4(S0 + row * N + ct * 16 + cq * 4);
    }
  }
  float uf[RT][kVJ];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = (wave * RT + rt) * 16 + r;
#pragma unroll
    for (int m = 0; m < kVJ; ++m) {
      const int j = cq + 4 * m;
      uf[rt][m] = (j < F) ? p.ring_u[(bh * L + (head + j) % L) * D + row] : 0.f;
    }
  }
  if (wave == 0) {
    const int j = lane;
    const float al = (j < F) ? p.ring_alpha[bh * L + (head + j) % L] : 1.f;
    float R = 1.f, P = 1.f;
    for (int m = 0; m < F; ++m) {
      const float am = __shfl(al, m, kWave);
      P *= am;
      if (m > j) R *= am;
    }
    if (j < F) s_w[j] = R;
    if (lane == 0) s_abar = P;
  }
  for (int t = tid; t < F * (N / 8); t += kBlock) {
    const int j = t / (N / 8), o = (t % (N / 8)) * 8;
    *reinterpret_cast<uint4*>(&s_k[j * N + o]) =
        ld_u4(p.ring_k + (((size_t)b * G + g) * L + (head + j) % L) * N + o);
  }
  __syncthreads();
  if (F > 0) fold_and_store<D, N, RT, NCT, kVJ>(S0, s, s_abar, s_k, s_w, uf, F, wave, r, cq);

  if (tid == 0) {
    if (h == 0) flag_error(p.err, bad);
    p.ptr[bh] = pack_ptr((head + F) % L, 0, rp.pending);
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
  p.ring_alpha = ring->decay;
  p.ptr = reinterpret_cast<unsigned long long*>(ring->ptr);
  p.err = ring->err;
  p.H = d->nheads;
  p.G = d->ngroups;
  p.L = d->capacity;
  return p;
}

template <int T>
int launch_gdn_verify(int D, const GdnReplayParams& p, dim3 grid, void* stream) {
  if (D == 64) return launch(gdn_verify_kernel<64, 128, T>, grid, dim3(kBlock), stream, p);
  return launch(gdn_verify_kernel<128, 128, T>, grid, dim3(kBlock), stream, p);
}

}  // namespace

extern "C" int gdn_decode_step(const rssm_dims* dims, float* state, const uint16_t* v,
                               const uint16_t* k, const uint16_t* q, const float* g,
                               const float* beta, float* y, void* stream) {
  if (!rssm_host::dims_ok(dims) || !state || !v || !k || !q || !g || !beta || !y) return RSSM_EINVAL;
  if (!rssm_host::shape_supported(dims)) return RSSM_ENOTSUP;
  GdnStdParams p{state, v, k, q, g, beta, y, dims->nheads, dims->ngroups};
  const dim3 grid(dims->batch * dims->nheads);
  if (dims->head_dim == 64) return launch(gdn_step_kernel<64, 128>, grid, dim3(kBlock), stream, p);
  return launch(gdn_step_kernel<128, 128>, grid, dim3(kBlock), stream, p);
}

extern "C" int gdn_replay_verify_T(const rssm_dims* dims, int32_t T, float* state0, rssm_ring* ring,
                                   const uint16_t* v, const uint16_t* k, const uint16_t* q,
                                   const float* g, const float* beta, float* y, int32_t* flushed,
                                   void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::ring_ok(ring, false) || !state0 || !v || !k || !q ||
      !g || !beta || !y)
    return RSSM_EINVAL;
  if (T < 1 || dims->capacity < 2 * T) return RSSM_EINVAL;
  if (!rssm_host::ring_shape_supported(dims) || T > kMaxT) return RSSM_ENOTSUP;
  GdnReplayParams p = make_gdn_params(dims, state0, ring);
  p.v = v;
  p.k = k;
  p.q = q;
  p.g = g;
  p.beta = beta;
  p.y = y;
  p.flushed = flushed;
  const dim3 grid(dims->batch * dims->nheads);
  const int D = dims->head_dim;
  switch (T) {
    case 1: return launch_gdn_verify<1>(D, p, grid, stream);
    case 2: return launch_gdn_verify<2>(D, p, grid, stream);
    case 3: return launch_gdn_verify<3>(D, p, grid, stream);
    case 4: return launch_gdn_verify<4>(D, p, grid, stream);
    case 5: return launch_gdn_verify<5>(D, p, grid, stream);
    case 6: return launch_gdn_verify<6>(D, p, grid, stream);
    case 7: return launch_gdn_verify<7>(D, p, grid, stream);
    default: return launch_gdn_verify<8>(D, p, grid, stream);
  }
}

extern "C" int gdn_replay_flush(const rssm_dims* dims, float* state0, rssm_ring* ring,
                                const int32_t* mask, void* stream) {
  if (!rssm_host::dims_ok(dims) || !rssm_host::ring_ok(ring, false) || !state0) return RSSM_EINVAL;
  if (dims->capacity < 1) return RSSM_EINVAL;
  if (!rssm_host::ring_shape_supported(dims)) return RSSM_ENOTSUP;
  GdnReplayParams p = make_gdn_params(dims, state0, ring);
  p.mask = mask;
  const dim3 grid(dims->batch * dims->nheads);
  if (dims->head_dim == 64) return launch(gdn_flush_kernel<64, 128>, grid, dim3(kBlock), stream, p);
  return launch(gdn_flush_kernel<128, 128>, grid, dim3(kBlock), stream, p);
}
