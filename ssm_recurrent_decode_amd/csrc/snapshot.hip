// The speculative-decoding baseline that ReplaySSM replaces, for Mamba-2 and
// Gated DeltaNet, and its device-side commit.
//
// Method: "ReplaySSM: Cache SSM Inputs, Not State" -- background ("the cost of
// summarising: a state cannot be undone": the usual workaround keeps one full
// state snapshot per draft and restores it on rejection) and algorithms
// ("speculative decoding", baseline bullet: serial state update per draft
// position, a full snapshot stored for every draft).
//
// Memory: every request owns P >= T + 1 state slots, pool [B, P, H, d, n] fp32,
// and an int32 index slot[b] naming the committed one.  A verify reads the
// committed slot once, runs the T drafts serially in registers and stores the
// state after draft s into slot (slot[b] + 1 + s) mod P.  Restoring the snapshot
// of the last accepted draft is then a move of slot[b], never a copy.  Per head
// and round the kernel streams 4dn bytes in and T * 4dn bytes out: the T-fold
// write traffic the pages charge to this route.
//
// Work decomposition and lane layout as the standard step kernels: one
// work-group of four waves per (request, head), the state in the tile layout of
// common.hpp, one float4 per 16 x 16 tile per lane.
#include "common.hpp"

namespace rssm {

struct SnapParams {
  float* pool;            // [B, P, H, D, N]
  const int32_t* slot;    // [B]
  const uint16_t* v;      // [B, T, H, D]
  const uint16_t* k;      // [B, T, G, N]
  const uint16_t* q;      // [B, T, G, N]
  const float* gate;      // Mamba-2: raw step dt [B, T, H]; GDN: log-decay g [B, T, H]
  const float* dt_bias;   // Mamba-2 [H]
  const float* A;         // Mamba-2 [H]
  const float* beta;      // GDN [B, T, H]
  float* y;               // [B, T, H, D]
  int32_t* err;
  int H, G, P;
};

// Index of the committed slot, reduced into [0, P) (flagged) when out of range.
__device__ __forceinline__ int committed_slot(const SnapParams& p, int b, bool report) {
  int cur = p.slot[b];
  if (cur < 0 || cur >= p.P) {
    cur %= p.P;
    if (cur < 0) cur += p.P;
    if (report) flag_error(p.err, RSSM_ERR_POINTERS);
  }
  return cur;
}

// T serial decode steps from the committed state; the state after draft s is
// stored to its own slot and y_s = S_s q_s.
//   Mamba-2: S <- a S + Delta v k^T,  Delta = softplus(dt + dt_bias), a = e^{A Delta}
//   GDN:     u = beta (v - e^g S k),  S <- e^g S + u k^T
template <int D, int N, int T, bool GDN>
__global__ __launch_bounds__(kBlock) void snapshot_verify_kernel(SnapParams p) {
  constexpr int NCT = N / 16;
  constexpr int RT = D / (16 * kWavesPerBlock);
  const int H = p.H, G = p.G, P = p.P;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);  // == b * H + h
  const int b = wg / H, h = wg - b * H, g = h / (H / G);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, cq = lane >> 4;

  const int cur = committed_slot(p, b, threadIdx.x == 0 && h == 0);
  const size_t slot_floats = (size_t)H * D * N;    // one slot of one request
  float* base = p.pool + (size_t)b * P * slot_floats + (size_t)h * D * N;

  float4 s[RT][NCT];  // line arrangement until each pair is settled (first draft)
  load_state_lines<N, RT, NCT>(s, base + (size_t)cur * slot_floats, wave, r, cq);

#pragma unroll
  for (int sd = 0; sd < T; ++sd) {
    const size_t bt = (size_t)b * T + sd;
    const uint16_t* kp = p.k + (bt * G + g) * N + cq * 4;
    const uint16_t* qp = p.q + (bt * G + g) * N + cq * 4;
    uint2 kk[NCT], qq[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      kk[ct] = ld_u2(kp + ct * 16);
      qq[ct] = ld_u2(qp + ct * 16);
    }
    float vr[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) vr[rt] = bf16_to_f32(p.v[(bt * H + h) * D + (wave * RT + rt) * 16 + r]);
    float decay, scale = 0.f;
    if constexpr (GDN) {
      decay = expf(p.gate[bt * H + h]);
      scale = p.beta[bt * H + h];
    } else {
      scale = softplus_f32(p.gate[bt * H + h] + p.dt_bias[h]);
      decay = expf(p.A[h] * scale);
    }
    int dst = cur + 1 + sd;  // < 2P because P >= T + 1
    if (dst >= P) dst -= P;
    float* Sd = base + (size_t)dst * slot_floats;

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = (wave * RT + rt) * 16 + r;
      float coef;  // the factor of k^T in the rank-1 update of this row
      if constexpr (GDN) {
        float sk = 0.f;
#pragma unroll
        for (int jj = 0; jj < NCT / 2; ++jj) {
          if (sd == 0) settle_pair(s[rt][2 * jj], s[rt][2 * jj + 1]);
          sk += dot4_bf16(s[rt][2 * jj], kk[2 * jj]) + dot4_bf16(s[rt][2 * jj + 1], kk[2 * jj + 1]);
        }
        sk = reduce_row4(sk);
        coef = scale * (vr[rt] - decay * sk);
      } else {
        coef = scale * vr[rt];
      }
      float acc = 0.f;
#pragma unroll
      for (int jj = 0; jj < NCT / 2; ++jj) {
        if (!GDN && sd == 0) settle_pair(s[rt][2 * jj], s[rt][2 * jj + 1]);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int ct = 2 * jj + half;
          float4 x = s[rt][ct];
          x.x = decay * x.x + coef * bf16_lo(kk[ct].x);
          x.y = decay * x.y + coef * bf16_hi(kk[ct].x);
          x.z = decay * x.z + coef * bf16_lo(kk[ct].y);
          x.w = decay * x.w + coef * bf16_hi(kk[ct].y);
          s[rt][ct] = x;
          acc += dot4_bf16(x, qq[ct]);
        }
        store_pair_lines<N>(Sd, wave * RT + rt, jj, s[rt][2 * jj], s[rt][2 * jj + 1], r, cq);
      }
      acc = reduce_row4(acc);
      if (cq == 0) p.y[(bt * H + h) * D + row] = acc;
    }
  }
}

struct CommitParams {
  int32_t* slot;
  const int32_t* accepted;
  int32_t* err;
  int B, T, P;
};

// slot[b] <- (slot[b] + clamp(accepted[b], 0, T)) mod P, one thread per request.
__global__ __launch_bounds__(kBlock) void snapshot_commit_kernel(CommitParams p) {
  const int b = blockIdx.x * kBlock + threadIdx.x;
  if (b >= p.B) return;
  int acc = p.accepted[b], cur = p.slot[b], bad = 0;
  if (acc < 0 || acc > p.T) {
    acc = acc < 0 ? 0 : p.T;
    bad |= RSSM_ERR_ACCEPTED;
  }
  if (cur < 0 || cur >= p.P) {
    cur %= p.P;
    if (cur < 0) cur += p.P;
    bad |= RSSM_ERR_POINTERS;
  }
  int nx = cur + acc;
  if (nx >= p.P) nx -= p.P;
  p.slot[b] = nx;
  flag_error(p.err, bad);
}

}  // namespace rssm

namespace {

using namespace rssm;

template <int D, int N, bool GDN>
int launch_snapshot(int T, const SnapParams& p, const dim3& grid, void* stream) {
  using rssm_host::launch;
  const dim3 blk(kBlock);
  switch (T) {
    case 1: return launch(snapshot_verify_kernel<D, N, 1, GDN>, grid, blk, stream, p);
    case 2: return launch(snapshot_verify_kernel<D, N, 2, GDN>, grid, blk, stream, p);
    case 3: return launch(snapshot_verify_kernel<D, N, 3, GDN>, grid, blk, stream, p);
    case 4: return launch(snapshot_verify_kernel<D, N, 4, GDN>, grid, blk, stream, p);
    case 5: return launch(snapshot_verify_kernel<D, N, 5, GDN>, grid, blk, stream, p);
    case 6: return launch(snapshot_verify_kernel<D, N, 6, GDN>, grid, blk, stream, p);
    case 7: return launch(snapshot_verify_kernel<D, N, 7, GDN>, grid, blk, stream, p);
    case 8: return launch(snapshot_verify_kernel<D, N, 8, GDN>, grid, blk, stream, p);
    default: return RSSM_ENOTSUP;
  }
}

int snapshot_common(const rssm_dims* dims, int32_t T, int32_t nslots, float* pool,
                    const int32_t* slot, const uint16_t* v, const uint16_t* k, const uint16_t* q,
                    bool gdn, SnapParams& p) {
  if (!rssm_host::dims_ok(dims) || !pool || !slot || !v || !k || !q || !rssm_host::aligned16(pool, slot, v, k, q))
    return RSSM_EINVAL;
  if (T < 1 || nslots < T + 1) return RSSM_EINVAL;
  (void)gdn;
  if (!rssm_host::shape_supported(dims) || T > kMaxT || (dims->flags & RSSM_F_Y_BF16)) return RSSM_ENOTSUP;
  p.pool = pool;
  p.slot = slot;
  p.v = v;
  p.k = k;
  p.q = q;
  p.H = dims->nheads;
  p.G = dims->ngroups;
  p.P = nslots;
  return RSSM_OK;
}

}  // namespace

extern "C" int ssm_snapshot_verify_T(const rssm_dims* dims, int32_t T, int32_t nslots, float* pool,
                                     const int32_t* slot, const uint16_t* v, const uint16_t* k,
                                     const uint16_t* q, const float* dt, const float* dt_bias,
                                     const float* A, float* y, int32_t* err, void* stream) {
  SnapParams p{};
  const int rc = snapshot_common(dims, T, nslots, pool, slot, v, k, q, false, p);
  if (rc != RSSM_OK) return rc;
  if (!dt || !dt_bias || !A || !y || !rssm_host::aligned16(dt, dt_bias, A, y)) return RSSM_EINVAL;
  p.gate = dt;
  p.dt_bias = dt_bias;
  p.A = A;
  p.y = y;
  p.err = err;
  const dim3 grid(dims->batch * dims->nheads);
  const bool d64 = dims->head_dim == 64;
  switch (dims->state_dim) {
    case 64: return d64 ? launch_snapshot<64, 64, false>(T, p, grid, stream) : launch_snapshot<128, 64, false>(T, p, grid, stream);
    case 256: return d64 ? launch_snapshot<64, 256, false>(T, p, grid, stream) : launch_snapshot<128, 256, false>(T, p, grid, stream);
    default: return d64 ? launch_snapshot<64, 128, false>(T, p, grid, stream) : launch_snapshot<128, 128, false>(T, p, grid, stream);
  }
}

extern "C" int gdn_snapshot_verify_T(const rssm_dims* dims, int32_t T, int32_t nslots, float* pool,
                                     const int32_t* slot, const uint16_t* v, const uint16_t* k,
                                     const uint16_t* q, const float* g, const float* beta, float* y,
                                     int32_t* err, void* stream) {
  SnapParams p{};
  const int rc = snapshot_common(dims, T, nslots, pool, slot, v, k, q, true, p);
  if (rc != RSSM_OK) return rc;
  if (!g || !beta || !y || !rssm_host::aligned16(g, beta, y)) return RSSM_EINVAL;
  p.gate = g;
  p.beta = beta;
  p.y = y;
  p.err = err;
  const dim3 grid(dims->batch * dims->nheads);
  const bool d64 = dims->head_dim == 64;
  switch (dims->state_dim) {
    case 64: return d64 ? launch_snapshot<64, 64, true>(T, p, grid, stream) : launch_snapshot<128, 64, true>(T, p, grid, stream);
    case 256: return d64 ? launch_snapshot<64, 256, true>(T, p, grid, stream) : launch_snapshot<128, 256, true>(T, p, grid, stream);
    default: return d64 ? launch_snapshot<64, 128, true>(T, p, grid, stream) : launch_snapshot<128, 128, true>(T, p, grid, stream);
  }
}

extern "C" int snapshot_commit(int32_t batch, int32_t T, int32_t nslots, int32_t* slot,
                               const int32_t* accepted, int32_t* err, void* stream) {
  if (batch < 1 || T < 1 || nslots < T + 1 || !slot || !accepted || !rssm_host::aligned16(slot, accepted) ||
      reinterpret_cast<uintptr_t>(err) % 4 != 0)
    return RSSM_EINVAL;
  CommitParams p{slot, accepted, err, batch, T, nslots};
  const dim3 grid((batch + kBlock - 1) / kBlock);
  return rssm_host::launch(snapshot_commit_kernel, grid, dim3(kBlock), stream, p);
}
